/* The C ABI used from plain C: no Python, no torch.  Builds small paged
 * pools in device memory, runs every data-movement call -- gather-scatter,
 * gather, scatter, the head-sliced copy, extract and rebuild -- on a HIP
 * stream, and compares every destination byte with the CPU oracle run on
 * host copies of the same bytes (the oracle is linked as test
 * infrastructure).  Also checks that a bad argument returns its status and
 * enqueues nothing.  Prints "abi_smoke ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvx.h"

/* oracle/kvx_oracle.c (test infrastructure) */
int64_t oracle_gather(int32_t Q, int64_t R, uint8_t* const* src_planes, int64_t src_stride,
                      int64_t src_page_stride, int32_t src_page_size, int64_t src_num_pages,
                      int32_t num_reqs, const int64_t* tok_off, const int64_t* src_pg_off,
                      const int32_t* src_ids, int64_t src_num_ids, uint8_t* staging,
                      int nthreads);
int64_t oracle_scatter(int32_t Q, int64_t R, const uint8_t* staging, int32_t num_reqs,
                       const int64_t* tok_off, const int64_t* dst_pg_off, const int32_t* dst_ids,
                       int64_t dst_num_ids, uint8_t* const* dst_planes, int64_t dst_stride,
                       int64_t dst_page_stride, int32_t dst_page_size, int64_t dst_num_pages,
                       int nthreads);
int64_t oracle_gather_scatter_heads(int32_t Q, int32_t nh, int64_t Db, uint8_t* const* src_planes,
                                    int64_t src_stride, int32_t src_page_size,
                                    int64_t src_num_pages, const int64_t* src_pg_off,
                                    const int32_t* src_ids, int64_t src_num_ids, int32_t src_H,
                                    int32_t src_h0, int32_t src_hnd, int32_t num_reqs,
                                    const int64_t* tok_off, uint8_t* const* dst_planes,
                                    int64_t dst_stride, int32_t dst_page_size,
                                    int64_t dst_num_pages, const int64_t* dst_pg_off,
                                    const int32_t* dst_ids, int64_t dst_num_ids, int32_t dst_H,
                                    int32_t dst_h0, int32_t dst_hnd, int nthreads);
int64_t oracle_extract_permute(int32_t Q, int32_t H, int64_t Db, uint8_t* const* hf_planes,
                               int64_t s_cap, int64_t seq, uint8_t* out, int nthreads);
int64_t oracle_rebuild_permute(int32_t Q, int32_t H, int64_t Db, const uint8_t* in, int64_t seq,
                               uint8_t* const* hf_planes, int64_t s_cap, int nthreads);
int64_t oracle_gather_scatter(int32_t Q, int64_t R, uint8_t* const* src_planes,
                              int64_t src_stride, int64_t src_page_stride, int32_t src_page_size,
                              int64_t src_num_pages, const int64_t* src_pg_off,
                              const int32_t* src_ids, int64_t src_num_ids, int32_t num_reqs,
                              const int64_t* tok_off, uint8_t* const* dst_planes,
                              int64_t dst_stride, int64_t dst_page_stride, int32_t dst_page_size,
                              int64_t dst_num_pages, const int64_t* dst_pg_off,
                              const int32_t* dst_ids, int64_t dst_num_ids, int nthreads);

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            return 2;                                                             \
        }                                                                         \
    } while (0)

#define CHECK_KVX(x)                                                              \
    do {                                                                          \
        kvx_status s_ = (x);                                                      \
        if (s_ != KVX_OK) {                                                       \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, kvx_status_str(s_)); \
            return 3;                                                             \
        }                                                                         \
    } while (0)

enum { L = 3, KV = 2, Q = L * KV, H = 4, D = 128, R = H * D * 2 };
enum { SRC_PAGE = 4, SRC_PAGES = 40, DST_PAGE = 16, DST_PAGES = 12, NREQ = 3 };

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 33);
}

static void shuffle(int32_t* a, int n) {
    for (int i = n - 1; i > 0; --i) {
        int j = (int)(next_u32() % (uint32_t)(i + 1));
        int32_t t = a[i]; a[i] = a[j]; a[j] = t;
    }
}

int main(void) {
    const int64_t lens[NREQ] = {37, 0, 61};          /* ragged, one empty request */
    int64_t tok_off[NREQ + 1] = {0};
    for (int r = 0; r < NREQ; ++r) tok_off[r + 1] = tok_off[r] + lens[r];
    const int64_t T = tok_off[NREQ];

    /* page tables: source pages from a permutation of 40, destination from 12 */
    int32_t sperm[SRC_PAGES], dperm[DST_PAGES];
    for (int i = 0; i < SRC_PAGES; ++i) sperm[i] = i;
    for (int i = 0; i < DST_PAGES; ++i) dperm[i] = i;
    shuffle(sperm, SRC_PAGES);
    shuffle(dperm, DST_PAGES);
    int64_t spg[NREQ + 1] = {0}, dpg[NREQ + 1] = {0};
    for (int r = 0; r < NREQ; ++r) {
        spg[r + 1] = spg[r] + (lens[r] + SRC_PAGE - 1) / SRC_PAGE;
        dpg[r + 1] = dpg[r] + (lens[r] + DST_PAGE - 1) / DST_PAGE;
    }
    const int64_t n_sids = spg[NREQ], n_dids = dpg[NREQ];

    const size_t splane = (size_t)SRC_PAGES * SRC_PAGE * R, dplane = (size_t)DST_PAGES * DST_PAGE * R;
    const size_t stage_bytes = (size_t)T * Q * R;
    uint8_t* src_h = malloc(Q * splane);
    uint8_t* dst_h = malloc(Q * dplane);
    uint8_t* exp_dst = malloc(Q * dplane);
    uint8_t* got_dst = malloc(Q * dplane);
    uint8_t* exp_st = calloc(stage_bytes, 1);
    uint8_t* got_st = malloc(stage_bytes);
    if (!src_h || !dst_h || !exp_dst || !got_dst || !exp_st || !got_st) return 4;
    for (size_t i = 0; i < Q * splane; ++i) src_h[i] = (uint8_t)next_u32();
    for (size_t i = 0; i < Q * dplane; ++i) dst_h[i] = (uint8_t)next_u32();

    uint8_t *src_d, *dst_d, *st_d;
    int64_t *tok_d, *spg_d, *dpg_d;
    int32_t *sid_d, *did_d;
    CHECK_HIP(hipMalloc((void**)&src_d, Q * splane));
    CHECK_HIP(hipMalloc((void**)&dst_d, Q * dplane));
    CHECK_HIP(hipMalloc((void**)&st_d, stage_bytes));
    CHECK_HIP(hipMalloc((void**)&tok_d, sizeof tok_off));
    CHECK_HIP(hipMalloc((void**)&spg_d, sizeof spg));
    CHECK_HIP(hipMalloc((void**)&dpg_d, sizeof dpg));
    CHECK_HIP(hipMalloc((void**)&sid_d, sizeof sperm));
    CHECK_HIP(hipMalloc((void**)&did_d, sizeof dperm));
    CHECK_HIP(hipMemcpy(src_d, src_h, Q * splane, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dst_d, dst_h, Q * dplane, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(st_d, 0, stage_bytes));
    CHECK_HIP(hipMemcpy(tok_d, tok_off, sizeof tok_off, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(spg_d, spg, sizeof spg, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dpg_d, dpg, sizeof dpg, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(sid_d, sperm, sizeof sperm, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(did_d, dperm, sizeof dperm, hipMemcpyHostToDevice));

    void* splanes[Q];
    void* dplanes[Q];
    uint8_t* splanes_h[Q];
    uint8_t* dplanes_h[Q];
    for (int q = 0; q < Q; ++q) {
        splanes[q] = src_d + q * splane;
        dplanes[q] = dst_d + q * dplane;
        splanes_h[q] = src_h + q * splane;
        dplanes_h[q] = exp_dst + q * dplane;
    }
    const kvx_layout lay = {L, KV, H, D, KVX_BF16};
    const kvx_pool sp = {splanes, SRC_PAGES, SRC_PAGE, R, 0};
    const kvx_pool dp = {dplanes, DST_PAGES, DST_PAGE, R, 0};
    const kvx_reqs reqs = {NREQ, T, tok_d};
    const kvx_table st = {spg_d, sid_d, n_sids};
    const kvx_table dt = {dpg_d, did_d, n_dids};
    unsigned long long* skipped_d;
    CHECK_HIP(hipMalloc((void**)&skipped_d, sizeof *skipped_d));
    CHECK_HIP(hipMemset(skipped_d, 0, sizeof *skipped_d));

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    if (kvx_abi_version() != KVX_ABI_VERSION) { fprintf(stderr, "ABI mismatch\n"); return 5; }
    /* a bad argument: a status, nothing enqueued */
    if (kvx_gather_scatter(NULL, &sp, &st, &reqs, &dp, &dt, skipped_d, stream) != KVX_E_NULL) {
        fprintf(stderr, "NULL layout not rejected\n");
        return 6;
    }
    CHECK_KVX(kvx_gather_scatter(&lay, &sp, &st, &reqs, &dp, &dt, skipped_d, stream));
    CHECK_KVX(kvx_gather(&lay, &sp, &st, &reqs, st_d, (int64_t)stage_bytes, skipped_d, 0, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    unsigned long long skipped = 1;
    CHECK_HIP(hipMemcpy(got_dst, dst_d, Q * dplane, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_st, st_d, stage_bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&skipped, skipped_d, sizeof skipped, hipMemcpyDeviceToHost));

    memcpy(exp_dst, dst_h, Q * dplane);
    int64_t s1 = oracle_gather_scatter(Q, R, splanes_h, R, 0, SRC_PAGE, SRC_PAGES, spg, sperm,
                                       SRC_PAGES, NREQ, tok_off, dplanes_h, R, 0, DST_PAGE,
                                       DST_PAGES, dpg, dperm, DST_PAGES, 1);
    int64_t s2 = oracle_gather(Q, R, splanes_h, R, 0, SRC_PAGE, SRC_PAGES, NREQ, tok_off, spg,
                               sperm, SRC_PAGES, exp_st, 1);
    if (memcmp(got_dst, exp_dst, Q * dplane) != 0) { fprintf(stderr, "gather_scatter differs\n"); return 7; }
    if (memcmp(got_st, exp_st, stage_bytes) != 0) { fprintf(stderr, "gather differs\n"); return 8; }
    if ((int64_t)skipped != s1 + s2 || skipped != 0) { fprintf(stderr, "skip count %llu\n", skipped); return 9; }
    /* the same gather with ordinary stores (KVX_OUT_CACHED), and an unknown flag refused */
    {
        uint8_t* st2_d;
        uint8_t* got2 = malloc(stage_bytes);
        if (!got2) return 4;
        CHECK_HIP(hipMalloc((void**)&st2_d, stage_bytes));
        CHECK_HIP(hipMemset(st2_d, 0, stage_bytes));
        if (kvx_gather(&lay, &sp, &st, &reqs, st2_d, (int64_t)stage_bytes, NULL, 2u, stream) !=
            KVX_E_UNSUPPORTED) {
            fprintf(stderr, "unknown flag not rejected\n");
            return 16;
        }
        CHECK_KVX(kvx_gather(&lay, &sp, &st, &reqs, st2_d, (int64_t)stage_bytes, NULL,
                             KVX_OUT_CACHED, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(got2, st2_d, stage_bytes, hipMemcpyDeviceToHost));
        if (memcmp(got2, exp_st, stage_bytes) != 0) { fprintf(stderr, "cached gather differs\n"); return 17; }
        CHECK_HIP(hipFree(st2_d));
        free(got2);
    }

    /* scatter the gathered staging into a third pool (destination layout) */
    {
        uint8_t* e_d;
        uint8_t* got = malloc(Q * dplane);
        uint8_t* exp = malloc(Q * dplane);
        uint8_t* eplanes_h[Q];
        void* eplanes[Q];
        if (!got || !exp) return 4;
        CHECK_HIP(hipMalloc((void**)&e_d, Q * dplane));
        CHECK_HIP(hipMemcpy(e_d, dst_h, Q * dplane, hipMemcpyHostToDevice));
        for (int q = 0; q < Q; ++q) { eplanes[q] = e_d + q * dplane; eplanes_h[q] = exp + q * dplane; }
        const kvx_pool ep = {eplanes, DST_PAGES, DST_PAGE, R, 0};
        CHECK_KVX(kvx_scatter(&lay, st_d, (int64_t)stage_bytes, &reqs, &ep, &dt, NULL, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(got, e_d, Q * dplane, hipMemcpyDeviceToHost));
        memcpy(exp, dst_h, Q * dplane);
        oracle_scatter(Q, R, got_st, NREQ, tok_off, dpg, dperm, DST_PAGES, eplanes_h, R, 0,
                       DST_PAGE, DST_PAGES, 1);
        if (memcmp(got, exp, Q * dplane) != 0) { fprintf(stderr, "scatter differs\n"); return 10; }
        hipFree(e_d); free(got); free(exp);
    }

    /* head-sliced copy: heads 1..2 of the 4-head source rows, read as HND
       pages of SRC_PAGE tokens, into 2-head NHD rows of a new pool */
    {
        enum { NH = 2, DB = D * 2 };
        const size_t hplane = (size_t)DST_PAGES * DST_PAGE * NH * DB;
        uint8_t* h_d;
        uint8_t* init = malloc(Q * hplane);
        uint8_t* got = malloc(Q * hplane);
        uint8_t* exp = malloc(Q * hplane);
        uint8_t* hplanes_h[Q];
        void* hplanes[Q];
        if (!init || !got || !exp) return 4;
        for (size_t i = 0; i < Q * hplane; ++i) init[i] = (uint8_t)next_u32();
        CHECK_HIP(hipMalloc((void**)&h_d, Q * hplane));
        CHECK_HIP(hipMemcpy(h_d, init, Q * hplane, hipMemcpyHostToDevice));
        for (int q = 0; q < Q; ++q) { hplanes[q] = h_d + q * hplane; hplanes_h[q] = exp + q * hplane; }
        const kvx_layout hl = {L, KV, NH, D, KVX_BF16};
        const kvx_pool hp = {hplanes, DST_PAGES, DST_PAGE, NH * DB, 0};
        const kvx_heads sh = {H, 1, KVX_HND}, dh = {NH, 0, KVX_NHD};
        CHECK_KVX(kvx_gather_scatter_heads(&hl, &sp, &st, &sh, &reqs, &hp, &dt, &dh, NULL, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(got, h_d, Q * hplane, hipMemcpyDeviceToHost));
        memcpy(exp, init, Q * hplane);
        oracle_gather_scatter_heads(Q, NH, DB, splanes_h, R, SRC_PAGE, SRC_PAGES, spg, sperm,
                                    SRC_PAGES, H, 1, 1, NREQ, tok_off, hplanes_h, NH * DB,
                                    DST_PAGE, DST_PAGES, dpg, dperm, DST_PAGES, NH, 0, 0, 1);
        if (memcmp(got, exp, Q * hplane) != 0) { fprintf(stderr, "heads differ\n"); return 11; }
        hipFree(h_d); free(init); free(got); free(exp);
    }

    /* extract [1][H][S_CAP][D] -> [Q][SEQ][H][D], then rebuild into fresh HF planes */
    {
        enum { S_CAP = 45, SEQ = 33, DB = D * 2 };
        const size_t hfp = (size_t)H * S_CAP * DB, flat = (size_t)Q * SEQ * H * DB;
        uint8_t* hf_h = malloc(Q * hfp);
        uint8_t* hf2_h = malloc(Q * hfp);
        uint8_t* exp_flat = calloc(flat, 1);
        uint8_t* got_flat = malloc(flat);
        uint8_t* exp_hf2 = malloc(Q * hfp);
        uint8_t* got_hf2 = malloc(Q * hfp);
        if (!hf_h || !hf2_h || !exp_flat || !got_flat || !exp_hf2 || !got_hf2) return 4;
        for (size_t i = 0; i < Q * hfp; ++i) { hf_h[i] = (uint8_t)next_u32(); hf2_h[i] = (uint8_t)next_u32(); }
        uint8_t *hf_d, *hf2_d, *flat_d;
        CHECK_HIP(hipMalloc((void**)&hf_d, Q * hfp));
        CHECK_HIP(hipMalloc((void**)&hf2_d, Q * hfp));
        CHECK_HIP(hipMalloc((void**)&flat_d, flat));
        CHECK_HIP(hipMemcpy(hf_d, hf_h, Q * hfp, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(hf2_d, hf2_h, Q * hfp, hipMemcpyHostToDevice));
        void* hfs[Q];
        void* hf2s[Q];
        uint8_t* hfs_h[Q];
        uint8_t* hf2s_h[Q];
        for (int q = 0; q < Q; ++q) {
            hfs[q] = hf_d + q * hfp; hf2s[q] = hf2_d + q * hfp;
            hfs_h[q] = hf_h + q * hfp; hf2s_h[q] = exp_hf2 + q * hfp;
        }
        CHECK_KVX(kvx_extract_permute(&lay, (const void* const*)hfs, S_CAP, SEQ, flat_d,
                                      (int64_t)flat, 0, stream));
        CHECK_KVX(kvx_rebuild_permute(&lay, flat_d, (int64_t)flat, SEQ, hf2s, S_CAP,
                                      KVX_OUT_CACHED, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(got_flat, flat_d, flat, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(got_hf2, hf2_d, Q * hfp, hipMemcpyDeviceToHost));
        oracle_extract_permute(Q, H, DB, hfs_h, S_CAP, SEQ, exp_flat, 1);
        memcpy(exp_hf2, hf2_h, Q * hfp);
        oracle_rebuild_permute(Q, H, DB, exp_flat, SEQ, hf2s_h, S_CAP, 1);
        if (memcmp(got_flat, exp_flat, flat) != 0) { fprintf(stderr, "extract differs\n"); return 12; }
        if (memcmp(got_hf2, exp_hf2, Q * hfp) != 0) { fprintf(stderr, "rebuild differs\n"); return 13; }
        hipFree(hf_d); hipFree(hf2_d); hipFree(flat_d);
        free(hf_h); free(hf2_h); free(exp_flat); free(got_flat); free(exp_hf2); free(got_hf2);
    }

    hipStreamDestroy(stream);
    hipFree(src_d); hipFree(dst_d); hipFree(st_d); hipFree(tok_d); hipFree(spg_d); hipFree(dpg_d);
    hipFree(sid_d); hipFree(did_d); hipFree(skipped_d);
    free(src_h); free(dst_h); free(exp_dst); free(got_dst); free(exp_st); free(got_st);
    printf("abi_smoke ok: %lld tokens, %d planes, rows of %d bytes, pages %d -> %d; "
           "gather_scatter, gather, scatter, heads, extract, rebuild\n",
           (long long)T, Q, R, SRC_PAGE, DST_PAGE);
    return 0;
}
