/* ep_c_caller.c -- a plain C99 caller of libep.so, with no Python and no torch.
 *
 * It shows that include/ep.h is a C header and that the library needs nothing
 * but device pointers, sizes and a stream: every buffer here comes from
 * hipMalloc, and the calls are the ones a C or C++ runtime would make.
 *
 *   ep_c_caller IN OUT
 *
 * IN (little-endian): int64 T; int32 H, k, E, R, P; then x [T*H] bf16 bits
 * (uint16), topk_idx [T*k] int64, topk_weights [T*k] float32.
 * The caller runs, on the null stream,
 *   ep_get_dispatch_layout -> ep_dispatch -> ep_combine (identity experts:
 *   the rows just dispatched) -> ep_dispatch_fp8 (when H % 128 == 0)
 * and writes to OUT, in this order: num_tokens_per_rank [R],
 * num_tokens_per_group [R/P], num_tokens_per_expert [E] (int32),
 * is_token_in_rank [T*R] (uint8), recv_expert_offset [E+1],
 * recv_rank_offset [R+1], token_row [T*k] (int32), int64 N (filled rows),
 * recv_src_idx [N] (int32), recv_topk_weights [N] (float32), recv_x [N*H]
 * (uint16), combined_x [T*H] (uint16), then, if H % 128 == 0, recv_x_fp8
 * [N*H] (uint8) and recv_scales [N*H/128] (float32).
 * Exit status 0 on success; otherwise a message on stderr and status 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"

static void die(const char* what) {
    fprintf(stderr, "ep_c_caller: %s\n", what);
    exit(1);
}

static void hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "ep_c_caller: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void ep_check(int status, const char* what) {
    if (status != EP_OK) {
        fprintf(stderr, "ep_c_caller: %s: %s (%s)\n", what, ep_status_string(status),
                ep_last_error());
        exit(1);
    }
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    hip_check(hipMalloc(&p, bytes > 0 ? bytes : 16), "hipMalloc");
    return p;
}

static void* host_alloc(size_t bytes) {
    void* p = malloc(bytes > 0 ? bytes : 16);
    if (!p) die("out of host memory");
    return p;
}

static void read_exact(FILE* f, void* dst, size_t bytes) {
    if (bytes > 0 && fread(dst, 1, bytes, f) != bytes) die("input file too short");
}

static void to_host_and_write(FILE* f, const void* dev, size_t bytes) {
    if (bytes == 0) return;
    void* h = host_alloc(bytes);
    hip_check(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H");
    if (fwrite(h, 1, bytes, f) != bytes) die("cannot write the output file");
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 3) die("usage: ep_c_caller IN OUT");
    FILE* in = fopen(argv[1], "rb");
    if (!in) die("cannot open the input file");
    int64_t T;
    int32_t hdr[5];
    read_exact(in, &T, sizeof T);
    read_exact(in, hdr, sizeof hdr);
    const int H = hdr[0], k = hdr[1], E = hdr[2], R = hdr[3], P = hdr[4];
    if (T < 0 || H < 8 || k < 1 || E < 1 || R < 1 || P < 1 || R % P != 0) die("bad header");
    const int G = R / P;
    const int64_t Tk = T * k;
    const size_t x_bytes = (size_t)(T * H) * sizeof(uint16_t);

    void* hx = host_alloc(x_bytes);
    int64_t* hidx = (int64_t*)host_alloc((size_t)Tk * sizeof(int64_t));
    float* hw = (float*)host_alloc((size_t)Tk * sizeof(float));
    read_exact(in, hx, x_bytes);
    read_exact(in, hidx, (size_t)Tk * sizeof(int64_t));
    read_exact(in, hw, (size_t)Tk * sizeof(float));
    fclose(in);

    void* x = dev_alloc(x_bytes);
    int64_t* idx = (int64_t*)dev_alloc((size_t)Tk * sizeof(int64_t));
    float* w = (float*)dev_alloc((size_t)Tk * sizeof(float));
    hip_check(hipMemcpy(x, hx, x_bytes, hipMemcpyHostToDevice), "hipMemcpy x");
    hip_check(hipMemcpy(idx, hidx, (size_t)Tk * sizeof(int64_t), hipMemcpyHostToDevice), "hipMemcpy idx");
    hip_check(hipMemcpy(w, hw, (size_t)Tk * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy w");

    /* layout */
    int32_t* per_rank = (int32_t*)dev_alloc((size_t)R * sizeof(int32_t));
    int32_t* per_group = (int32_t*)dev_alloc((size_t)G * sizeof(int32_t));
    int32_t* per_expert = (int32_t*)dev_alloc((size_t)E * sizeof(int32_t));
    uint8_t* in_rank = (uint8_t*)dev_alloc((size_t)(T * R));
    const size_t ws_l_bytes = ep_layout_workspace_bytes(T, E, R, P);
    void* ws_l = dev_alloc(ws_l_bytes);
    ep_check(ep_get_dispatch_layout(idx, T, k, E, R, P, per_rank, per_group, per_expert, in_rank,
                                    ws_l, ws_l_bytes, NULL),
             "ep_get_dispatch_layout");

    /* dispatch: receive buffers at capacity T*k rows */
    void* recv_x = dev_alloc((size_t)Tk * H * sizeof(uint16_t));
    int32_t* src = (int32_t*)dev_alloc((size_t)Tk * sizeof(int32_t));
    float* recv_w = (float*)dev_alloc((size_t)Tk * sizeof(float));
    int32_t* eoff = (int32_t*)dev_alloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* roff = (int32_t*)dev_alloc((size_t)(R + 1) * sizeof(int32_t));
    int32_t* token_row = (int32_t*)dev_alloc((size_t)Tk * sizeof(int32_t));
    const size_t ws_d_bytes = ep_dispatch_workspace_bytes(T, k, E);
    void* ws_d = dev_alloc(ws_d_bytes);
    ep_check(ep_dispatch(x, idx, w, T, H, k, E, R, recv_x, src, recv_w, eoff, roff, token_row,
                         ws_d, ws_d_bytes, NULL),
             "ep_dispatch");

    /* combine over the dispatched rows (identity experts) */
    void* out = dev_alloc(x_bytes);
    ep_check(ep_combine(recv_x, Tk, token_row, w, T, H, k, out, NULL), "ep_combine");

    /* FP8 dispatch */
    uint8_t* q = NULL;
    float* scales = NULL;
    if (H % 128 == 0) {
        q = (uint8_t*)dev_alloc((size_t)Tk * H);
        scales = (float*)dev_alloc((size_t)Tk * (H / 128) * sizeof(float));
        int32_t* src8 = (int32_t*)dev_alloc((size_t)Tk * sizeof(int32_t));
        float* w8 = (float*)dev_alloc((size_t)Tk * sizeof(float));
        int32_t* eoff8 = (int32_t*)dev_alloc((size_t)(E + 1) * sizeof(int32_t));
        int32_t* tr8 = (int32_t*)dev_alloc((size_t)Tk * sizeof(int32_t));
        ep_check(ep_dispatch_fp8(x, idx, w, T, H, k, E, R, q, scales, src8, w8, eoff8, NULL, tr8,
                                 ws_d, ws_d_bytes, NULL),
                 "ep_dispatch_fp8");
    }
    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

    int32_t* heoff = (int32_t*)host_alloc((size_t)(E + 1) * sizeof(int32_t));
    hip_check(hipMemcpy(heoff, eoff, (size_t)(E + 1) * sizeof(int32_t), hipMemcpyDeviceToHost),
              "hipMemcpy offsets");
    const int64_t N = heoff[E];
    if (N < 0 || N > Tk) die("filled row count out of range");

    FILE* o = fopen(argv[2], "wb");
    if (!o) die("cannot open the output file");
    to_host_and_write(o, per_rank, (size_t)R * sizeof(int32_t));
    to_host_and_write(o, per_group, (size_t)G * sizeof(int32_t));
    to_host_and_write(o, per_expert, (size_t)E * sizeof(int32_t));
    to_host_and_write(o, in_rank, (size_t)(T * R));
    to_host_and_write(o, eoff, (size_t)(E + 1) * sizeof(int32_t));
    to_host_and_write(o, roff, (size_t)(R + 1) * sizeof(int32_t));
    to_host_and_write(o, token_row, (size_t)Tk * sizeof(int32_t));
    if (fwrite(&N, sizeof N, 1, o) != 1) die("cannot write the output file");
    to_host_and_write(o, src, (size_t)N * sizeof(int32_t));
    to_host_and_write(o, recv_w, (size_t)N * sizeof(float));
    to_host_and_write(o, recv_x, (size_t)N * H * sizeof(uint16_t));
    to_host_and_write(o, out, x_bytes);
    if (H % 128 == 0) {
        to_host_and_write(o, q, (size_t)N * H);
        to_host_and_write(o, scales, (size_t)N * (H / 128) * sizeof(float));
    }
    if (fclose(o) != 0) die("cannot close the output file");
    return 0;
}
