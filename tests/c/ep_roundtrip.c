/*
 * ep_roundtrip.c -- drives libep.so from plain C through include/ep.h alone
 * (test infrastructure).  A small routing with distinct experts per token and
 * weights that sum to exactly one; the expert stage is the identity (the
 * receive rows are the expert outputs), so with bf16 dispatch the combine must
 * return every token bit for bit (the stage table's round trip: dispatch
 * arranges tokens by expert, combine brings them back with a weighted sum).
 * Also checks that the per-expert counts sum to T*k and that the slots are a
 * bijection onto the receive rows.  Exit status 0 on success.
 */
#ifndef __HIP_PLATFORM_AMD__
#define __HIP_PLATFORM_AMD__ 1
#endif
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            return 2;                                                                \
        }                                                                            \
    } while (0)
#define CHECK_EP(call)                                                               \
    do {                                                                             \
        int s_ = (call);                                                             \
        if (s_ != EP_OK) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, ep_status_string(s_));         \
            return 3;                                                                \
        }                                                                            \
    } while (0)

static uint32_t lcg(uint32_t* s) {
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

int main(void) {
    const int64_t T = 300;
    const int32_t k = 4, E = 32, G = 4, H = 512;
    const int64_t P = T * k;
    uint32_t seed = 12345u;

    int64_t* idx = malloc(sizeof(int64_t) * P);
    float* w = malloc(sizeof(float) * P);
    uint16_t* x = malloc(sizeof(uint16_t) * T * H);
    uint16_t* out = malloc(sizeof(uint16_t) * T * H);
    int32_t* slot = malloc(sizeof(int32_t) * P);
    int32_t counts[32], flags = -1;
    const float wj[4] = {0.5f, 0.25f, 0.125f, 0.125f};  /* sum exactly 1 */
    if (!idx || !w || !x || !out || !slot) return 4;
    for (int64_t t = 0; t < T; ++t) {
        int32_t base = (int32_t)(lcg(&seed) % (uint32_t)E);
        for (int32_t j = 0; j < k; ++j) {
            idx[t * k + j] = (base + j * (E / k)) % E;      /* k distinct experts */
            w[t * k + j] = wj[j];
        }
    }
    for (int64_t i = 0; i < T * H; ++i) {                    /* bf16 in +-[1, 2) */
        uint32_t r = lcg(&seed);
        x[i] = (uint16_t)(0x3F80u | (r & 0x7Fu) | ((r >> 7) & 1u) << 15);
    }

    ep_layout_t L;
    CHECK_EP(ep_layout_init(&L, T, k, E, G, 0));
    const int64_t R = L.num_recv_rows;
    const size_t ws_bytes = ep_layout_workspace_bytes(T, k, E);
    void *d_idx, *d_w, *d_x, *d_recv, *d_out, *d_ws;
    int32_t *d_cnt, *d_off, *d_grp, *d_slot, *d_flags;
    CHECK_HIP(hipMalloc(&d_idx, sizeof(int64_t) * P));
    CHECK_HIP(hipMalloc(&d_w, sizeof(float) * P));
    CHECK_HIP(hipMalloc(&d_x, sizeof(uint16_t) * T * H));
    CHECK_HIP(hipMalloc(&d_recv, sizeof(uint16_t) * R * H));
    CHECK_HIP(hipMalloc(&d_out, sizeof(uint16_t) * T * H));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMalloc((void**)&d_cnt, sizeof(int32_t) * E));
    CHECK_HIP(hipMalloc((void**)&d_off, sizeof(int32_t) * (E + 1)));
    CHECK_HIP(hipMalloc((void**)&d_grp, sizeof(int32_t) * G));
    CHECK_HIP(hipMalloc((void**)&d_slot, sizeof(int32_t) * P));
    CHECK_HIP(hipMalloc((void**)&d_flags, sizeof(int32_t)));
    CHECK_HIP(hipMemcpy(d_idx, idx, sizeof(int64_t) * P, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, sizeof(float) * P, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));
    L.num_tokens_per_expert = d_cnt;
    L.expert_offsets = d_off;
    L.num_tokens_per_group = d_grp;
    L.slot_idx = d_slot;
    L.recv_src = NULL;
    L.error_flags = d_flags;

    CHECK_EP(ep_get_layout(d_idx, &L, d_ws, ws_bytes, NULL));
    CHECK_EP(ep_dispatch(d_x, &L, H, EP_BF16, d_recv, NULL, NULL));
    CHECK_EP(ep_combine(d_recv, d_w, &L, H, d_out, NULL));  /* identity experts */
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot, d_slot, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_cnt, sizeof(int32_t) * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&flags, d_flags, sizeof(int32_t), hipMemcpyDeviceToHost));

    int bad = 0;
    int64_t total = 0;
    for (int32_t e = 0; e < E; ++e) total += counts[e];
    if (flags != 0 || total != P) bad |= 1;
    unsigned char* seen = calloc((size_t)R, 1);
    if (!seen) return 4;
    for (int64_t p = 0; p < P; ++p) {
        if (slot[p] < 0 || slot[p] >= R || seen[slot[p]]) { bad |= 2; break; }
        seen[slot[p]] = 1;
    }
    if (memcmp(out, x, sizeof(uint16_t) * T * H) != 0) bad |= 4;
    printf("ep_roundtrip: %s (T=%lld k=%d E=%d H=%d; %s)\n", bad ? "FAILED" : "ok", (long long)T, k,
           E, H, ep_version());
    free(seen);
    hipFree(d_idx); hipFree(d_w); hipFree(d_x); hipFree(d_recv); hipFree(d_out); hipFree(d_ws);
    hipFree(d_cnt); hipFree(d_off); hipFree(d_grp); hipFree(d_slot); hipFree(d_flags);
    free(idx); free(w); free(x); free(out); free(slot);
    return bad ? 1 : 0;
}
