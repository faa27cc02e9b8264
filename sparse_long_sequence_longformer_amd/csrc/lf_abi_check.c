/*
 * A plain C caller of liblfattn.so: no C++, no Python, no torch.  It reads one problem
 * from a file, runs lf_attn_forward on the GPU through the C-ABI with device memory of
 * its own, and writes the output to a file.
 *
 * Input file (little-endian): int32 B, H, L, d_h, w, n_global, has_pad; int32
 * dil[H]; int32 global_idx[n_global]; uint8 pad[B][L] if has_pad; then q, k, v as
 * bf16 [B][H][L][d_h] each.  Output file: the bf16 output, same layout.
 *
 * Usage: lf_abi_check IN OUT.  Exit status 0 on success; otherwise the status and
 * message of the failing call are printed and the status is the exit code.  With a
 * third argument "bad-w", the call is made with w = -1 instead and must fail with
 * LF_ERR_INVALID_ARG before anything is enqueued (exit 0 when it does).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lf_attn.h"

static int read_all(FILE* f, void* dst, size_t n) { return fread(dst, 1, n, f) == n; }

int main(int argc, char** argv) {
    if (argc < 3) {
        fprintf(stderr, "usage: %s IN OUT [bad-w]\n", argv[0]);
        return 2;
    }
    const int bad_w = argc > 3 && strcmp(argv[3], "bad-w") == 0;
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 2;
    }
    int32_t hdr[7];
    if (!read_all(in, hdr, sizeof(hdr))) return 2;
    const int B = hdr[0], H = hdr[1], L = hdr[2], d = hdr[3], w = hdr[4], ng = hdr[5], has_pad = hdr[6];
    if (B < 1 || H < 1 || H > LF_MAX_HEADS || L < 1 || d != LF_HEAD_DIM || ng < 0 || ng > LF_MAX_GLOBALS) {
        fprintf(stderr, "bad header\n");
        return 2;
    }
    int32_t dil[LF_MAX_HEADS], gidx[LF_MAX_GLOBALS];
    if (!read_all(in, dil, sizeof(int32_t) * (size_t)H) || !read_all(in, gidx, sizeof(int32_t) * (size_t)ng))
        return 2;
    const size_t n = (size_t)B * H * L * d, bytes = n * sizeof(uint16_t), pbytes = (size_t)B * L;
    uint8_t* pad = has_pad ? (uint8_t*)malloc(pbytes) : NULL;
    uint16_t* host = (uint16_t*)malloc(3 * bytes);
    if (!host || (has_pad && !pad)) return 2;
    if ((has_pad && !read_all(in, pad, pbytes)) || !read_all(in, host, 3 * bytes)) {
        fprintf(stderr, "short input file\n");
        return 2;
    }
    fclose(in);

    void *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL, *dpad = NULL;
    if (hipMalloc(&dq, bytes) != hipSuccess || hipMalloc(&dk, bytes) != hipSuccess ||
        hipMalloc(&dv, bytes) != hipSuccess || hipMalloc(&dout, bytes) != hipSuccess ||
        (has_pad && hipMalloc(&dpad, pbytes) != hipSuccess)) {
        fprintf(stderr, "hipMalloc failed\n");
        return 3;
    }
    if (hipMemcpy(dq, host, bytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dk, host + n, bytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dv, host + 2 * n, bytes, hipMemcpyHostToDevice) != hipSuccess ||
        (has_pad && hipMemcpy(dpad, pad, pbytes, hipMemcpyHostToDevice) != hipSuccess)) {
        fprintf(stderr, "hipMemcpy to the device failed\n");
        return 3;
    }

    lf_attn_t h = NULL;
    lf_status st = lf_attn_create(&h, LF_BF16);
    if (st != LF_OK) {
        fprintf(stderr, "lf_attn_create: %s\n", lf_attn_status_string(st));
        return (int)st;
    }
    st = lf_attn_forward(h, dq, dk, dv, dout, B, H, L, d, bad_w ? -1 : w, dil, ng ? gidx : NULL, ng,
                         (const uint8_t*)dpad, NULL);
    if (bad_w) {
        const int ok = st == LF_ERR_INVALID_ARG;
        printf("bad w: %s (%s)\n", lf_attn_status_string(st), lf_attn_last_error(h));
        lf_attn_destroy(h);
        return ok ? 0 : 1;
    }
    if (st != LF_OK) {
        fprintf(stderr, "lf_attn_forward: %s (%s)\n", lf_attn_status_string(st), lf_attn_last_error(h));
        return (int)st;
    }
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(host, dout, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        fprintf(stderr, "the forward or the copy back failed\n");
        return 3;
    }
    st = lf_attn_destroy(h);
    if (st != LF_OK) {
        fprintf(stderr, "lf_attn_destroy: %s\n", lf_attn_status_string(st));
        return (int)st;
    }
    FILE* out = fopen(argv[2], "wb");
    if (!out || fwrite(host, 1, bytes, out) != bytes) {
        fprintf(stderr, "cannot write %s\n", argv[2]);
        return 2;
    }
    fclose(out);
    (void)hipFree(dq);
    (void)hipFree(dk);
    (void)hipFree(dv);
    (void)hipFree(dout);
    if (dpad) (void)hipFree(dpad);
    free(host);
    free(pad);
    printf("ok B=%d H=%d L=%d w=%d n_global=%d\n", B, H, L, w, ng);
    return 0;
}
