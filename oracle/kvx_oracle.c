/*
 * kvx_oracle.c -- CPU oracle for the paged-KV data-movement path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code, no
 * header and no constant with the HIP library; it is a plain, slow,
 * obviously-correct row-by-row memcpy loop over the slot tables.
 *
 * Sources (the pages' titles and the sections used):
 *   [budget]  "穷人版 PD 分离：在消费级显卡上把 TTS 推理拆成两半" (kilerd.me,
 *             pd-on-a-budget): sections "B300：让 P 直接写 D 的显存" and
 *             "5090：一个看得见所有卡的代理", plus its failure-handling section.
 *   [mini]    "mini-infer系统实战-18-PD 解耦：把 Prefill 和 Decode 拆进两个进程之后
 *             发生了什么" (smarter.xin): section "KV 序列化格式选择".
 *   [survey]  "PD分离调研：从推理阶段拆分到Mooncake的KVCache中心架构"
 *             (gentlecold.top): sections 7.4 (registering the per-layer KV
 *             cache addresses), 7.6 (P writes KV blocks into D) and 7.7
 *             (the transfer plan for P and D with different TP sizes).
 *
 * What it computes (every function is a bitwise copy; no arithmetic touches
 * the KV values, so fp16 / bf16 / NaN payloads pass through unchanged):
 *
 *   Token-paged pool ([budget], 5090 section).  The pool is paged per token,
 *   so one request's KV is spread over the pool in thousands of pieces of a
 *   few KB, and a freshly started pool yields one contiguous block per
 *   (layer, K/V).  A pool is therefore read as Q planes (Q = layers x {K,V}),
 *   each an array of slots of R bytes (R = kv_heads * head_dim * element
 *   size); slot s of plane q sits at planes[q] + s*stride.
 *
 *   Paged blocks ([survey] 7.4).  Each per-layer cache tensor is cut into
 *   num_blocks equal blocks of block_len bytes.  With B tokens per page,
 *   token t of request r lives in page ids[pg_off[r] + t/B], row t%B of it.
 *   Page p of plane q starts at planes[q] + p*page_stride and its row i at
 *   another i*stride bytes.  When a block holds only one plane's B rows,
 *   page_stride = B*stride (0 selects this) and the row is slot p*B + t%B;
 *   when a tensor's blocks hold K and V (or all layers) together,
 *   page_stride is the block length and the planes' bases differ by where
 *   their rows sit inside a block.
 *
 *   Gather / scatter ([budget], 5090 section).  P first collects the rows to
 *   be sent into one contiguous staging area, one transfer moves it, and D
 *   writes the rows back into its own pages.  The staging layout is the
 *   per-layer (k, v) list of [seq, kv_heads, head_dim] tensors of [mini],
 *   laid end to end: request r starts at token offset tok_off[r] and holds,
 *   plane by plane, its n_r rows.  Byte offset of (r, q, t):
 *       (tok_off[r] * Q + q * n_r + t) * R.
 *
 *   Gather-scatter ([budget], B300 section; [survey] 7.6).  Each scattered
 *   source row is written straight into its destination page, with no
 *   staging in between.
 *
 *   Extract / rebuild permute ([mini]).  Extract keeps batch 0 and the first
 *   seq_len positions of a [1, H, S, D] layer cache and swaps the head and
 *   sequence axes, giving [seq, H, D]; rebuild swaps them back into
 *   [1, H, seq, D].  The Q per-plane [seq, H, D] results are stacked as one
 *   [Q][seq][H][D] buffer.
 *
 *   Page-table reads.  Token t of request r takes its page id from entry
 *   pg_off[r] + t/B of the side's page-id array of num_ids entries: a
 *   request's list is read from its start onward, one entry per page of its
 *   tokens, and the start of the next request's list is never consulted (a
 *   list shorter than its tokens need runs on into the entries after it).
 *
 *   Out-of-range rows.  A row whose table index pg_off[r] + t/B falls outside
 *   [0, num_ids), or whose page id falls outside [0, num_pages), is never
 *   dereferenced: it is skipped, counted, and its destination bytes keep their
 *   prior contents ([budget], failure-handling section: the failure to rule
 *   out is a late write landing in pages already handed to someone else, so
 *   nothing outside the pool may be addressed, whatever the tables say).
 *
 * Every function returns the number of skipped rows (>= 0).  Work may be
 * split over nthreads POSIX threads by (request, plane) pairs; the result does
 * not depend on nthreads because no two pairs write the same byte under the
 * precondition that destination rows are distinct.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- tables -- */

/* A pool side of a move: Q plane base pointers, row and page strides, paging. */
typedef struct {
    uint8_t* const* planes;
    int64_t stride;         /* bytes between consecutive rows of a page */
    int64_t page_stride;    /* bytes between consecutive pages of a plane */
    int32_t page_size;
    int64_t num_pages;
    const int64_t* pg_off;
    const int32_t* ids;
    int64_t num_ids;        /* entries of ids */
} pool_side;

/* Page id of token t of request r, or -1 when its table index or the id it
 * holds is out of range.  The index pg_off[r] + t/B is a plain integer: its
 * range is checked before the sum is formed, so no pg_off value makes it
 * wrap (t/B >= 0 and num_ids >= 0, so neither bound overflows). */
static int64_t page_of(const pool_side* s, int64_t r, int64_t t)
{
    int64_t k = t / s->page_size;
    if (s->pg_off[r] < -k || s->pg_off[r] >= s->num_ids - k) return -1;
    int64_t idx = s->pg_off[r] + k;
    int64_t page = (int64_t)s->ids[idx];
    if (page < 0 || page >= s->num_pages) return -1;
    return page;
}

/* Byte offset from its plane's base of token t of request r, or -1 when the
 * row is out of range. */
static int64_t row_offset(const pool_side* s, int64_t r, int64_t t)
{
    int64_t page = page_of(s, r, t);
    if (page < 0) return -1;
    return page * s->page_stride + (t % s->page_size) * s->stride;
}

/* page_stride 0 stands for page_size * stride: pages of one plane's rows only. */
static int64_t page_stride_of(int64_t page_stride, int32_t page_size, int64_t stride)
{
    return page_stride != 0 ? page_stride : (int64_t)page_size * stride;
}

enum { OP_GATHER = 0, OP_SCATTER = 1, OP_GATHER_SCATTER = 2 };

typedef struct {
    int op;
    int32_t Q;
    int64_t R;
    int32_t num_reqs;
    const int64_t* tok_off;
    pool_side src, dst;
    uint8_t* staging;       /* gather: destination; scatter: source */
    int64_t first_pair, last_pair;   /* (r, q) pairs [first, last) */
    int64_t skipped;
} row_job;

static void* run_rows(void* arg)
{
    row_job* j = (row_job*)arg;
    int64_t skipped = 0;
    for (int64_t pair = j->first_pair; pair < j->last_pair; ++pair) {
        int64_t r = pair / j->Q;
        int64_t q = pair % j->Q;
        int64_t n = j->tok_off[r + 1] - j->tok_off[r];
        for (int64_t t = 0; t < n; ++t) {
            uint8_t* staged = j->staging
                ? j->staging + (j->tok_off[r] * j->Q + q * n + t) * j->R : NULL;
            if (j->op == OP_GATHER) {
                int64_t s = row_offset(&j->src, r, t);
                if (s < 0) { ++skipped; continue; }
                memcpy(staged, j->src.planes[q] + s, (size_t)j->R);
            } else if (j->op == OP_SCATTER) {
                int64_t d = row_offset(&j->dst, r, t);
                if (d < 0) { ++skipped; continue; }
                memcpy(j->dst.planes[q] + d, staged, (size_t)j->R);
            } else {
                int64_t s = row_offset(&j->src, r, t);
                int64_t d = row_offset(&j->dst, r, t);
                if (s < 0 || d < 0) { ++skipped; continue; }
                memcpy(j->dst.planes[q] + d, j->src.planes[q] + s, (size_t)j->R);
            }
        }
    }
    j->skipped = skipped;
    return NULL;
}

/* Split the (request, plane) pairs over nthreads threads and run them. */
static int64_t run_split(row_job proto, int nthreads)
{
    int64_t pairs = (int64_t)proto.num_reqs * proto.Q;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (pairs < nthreads) nthreads = pairs > 0 ? (int)pairs : 1;
    row_job jobs[256];
    pthread_t tids[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].first_pair = pairs * i / nthreads;
        jobs[i].last_pair = pairs * (i + 1) / nthreads;
        jobs[i].skipped = 0;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&tids[i], NULL, run_rows, &jobs[i]) == 0;
    run_rows(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(tids[i], NULL);
        else run_rows(&jobs[i]);
    }
    int64_t total = 0;
    for (int i = 0; i < nthreads; ++i) total += jobs[i].skipped;
    return total;
}

/* Gather: staging(r, q, t) <- src plane q, row of token t of request r. */
int64_t oracle_gather(int32_t Q, int64_t R,
                      uint8_t* const* src_planes, int64_t src_stride, int64_t src_page_stride,
                      int32_t src_page_size, int64_t src_num_pages,
                      int32_t num_reqs, const int64_t* tok_off,
                      const int64_t* src_pg_off, const int32_t* src_ids, int64_t src_num_ids,
                      uint8_t* staging, int nthreads)
{
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = OP_GATHER; j.Q = Q; j.R = R; j.num_reqs = num_reqs; j.tok_off = tok_off;
    j.src.planes = src_planes; j.src.stride = src_stride; j.src.page_size = src_page_size;
    j.src.page_stride = page_stride_of(src_page_stride, src_page_size, src_stride);
    j.src.num_pages = src_num_pages; j.src.pg_off = src_pg_off; j.src.ids = src_ids;
    j.src.num_ids = src_num_ids;
    j.staging = staging;
    return run_split(j, nthreads);
}

/* Scatter: dst plane q, row of token t of request r <- staging(r, q, t). */
int64_t oracle_scatter(int32_t Q, int64_t R, const uint8_t* staging,
                       int32_t num_reqs, const int64_t* tok_off,
                       const int64_t* dst_pg_off, const int32_t* dst_ids, int64_t dst_num_ids,
                       uint8_t* const* dst_planes, int64_t dst_stride, int64_t dst_page_stride,
                       int32_t dst_page_size, int64_t dst_num_pages, int nthreads)
{
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = OP_SCATTER; j.Q = Q; j.R = R; j.num_reqs = num_reqs; j.tok_off = tok_off;
    j.dst.planes = dst_planes; j.dst.stride = dst_stride; j.dst.page_size = dst_page_size;
    j.dst.page_stride = page_stride_of(dst_page_stride, dst_page_size, dst_stride);
    j.dst.num_pages = dst_num_pages; j.dst.pg_off = dst_pg_off; j.dst.ids = dst_ids;
    j.dst.num_ids = dst_num_ids;
    j.staging = (uint8_t*)staging;
    return run_split(j, nthreads);
}

/* Gather-scatter: dst plane q at the dst row of (r, t) <- src plane q at the
 * src row of (r, t).  Both sides share the token CSR tok_off; each has its
 * own page table, page size and strides.  A token out of range on either
 * side is skipped (and counted) in every plane. */
int64_t oracle_gather_scatter(int32_t Q, int64_t R,
                              uint8_t* const* src_planes, int64_t src_stride,
                              int64_t src_page_stride, int32_t src_page_size,
                              int64_t src_num_pages,
                              const int64_t* src_pg_off, const int32_t* src_ids,
                              int64_t src_num_ids,
                              int32_t num_reqs, const int64_t* tok_off,
                              uint8_t* const* dst_planes, int64_t dst_stride,
                              int64_t dst_page_stride, int32_t dst_page_size,
                              int64_t dst_num_pages,
                              const int64_t* dst_pg_off, const int32_t* dst_ids,
                              int64_t dst_num_ids, int nthreads)
{
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = OP_GATHER_SCATTER; j.Q = Q; j.R = R; j.num_reqs = num_reqs; j.tok_off = tok_off;
    j.src.planes = src_planes; j.src.stride = src_stride; j.src.page_size = src_page_size;
    j.src.page_stride = page_stride_of(src_page_stride, src_page_size, src_stride);
    j.src.num_pages = src_num_pages; j.src.pg_off = src_pg_off; j.src.ids = src_ids;
    j.src.num_ids = src_num_ids;
    j.dst.planes = dst_planes; j.dst.stride = dst_stride; j.dst.page_size = dst_page_size;
    j.dst.page_stride = page_stride_of(dst_page_stride, dst_page_size, dst_stride);
    j.dst.num_pages = dst_num_pages; j.dst.pg_off = dst_pg_off; j.dst.ids = dst_ids;
    j.dst.num_ids = dst_num_ids;
    return run_split(j, nthreads);
}

/* ---------------------------------------------------- head-sliced copies -- */

/* Head-sliced gather-scatter ([survey] 7.7).  When P and D run with different
 * tensor-parallel sizes, a rank holds kv_heads / tp heads of every row, and a
 * P rank and a D rank move only the heads they share: a contiguous head range
 * that starts at one head in the source rows and at another in the
 * destination rows.  The same section notes that non-MLA models then keep
 * each block head-major (HND), which makes one head of one block contiguous.
 *
 * A pool side: H heads per token row, the slice starts at head h0, and a page
 * of B tokens is laid out token-major (NHD: [B][H][D]) or head-major (HND:
 * [H][B][D]); stride is the bytes of one token row (H * Db when dense), so a
 * page spans B * stride bytes.  Byte offset of head h of token t in a page:
 *     NHD: (page * B + t % B) * stride + h * Db
 *     HND: page * B * stride + (h * B + t % B) * Db
 * For every request r, plane q, token t < n_r and j < nh, the Db bytes of
 * source head h0_src + j go to destination head h0_dst + j.  A token whose
 * page id is out of range on either side is skipped (all nh heads) and
 * counted once. */
typedef struct {
    uint8_t* const* planes;
    int64_t stride;
    int32_t page_size;
    int64_t num_pages;
    const int64_t* pg_off;
    const int32_t* ids;
    int64_t num_ids;
    int32_t H, h0, hnd;
} head_side;

typedef struct {
    int32_t Q, nh;
    int64_t Db;
    int32_t num_reqs;
    const int64_t* tok_off;
    head_side src, dst;
    int64_t first_pair, last_pair;
    int64_t skipped;
} head_job;

/* Byte offset of head h of token t of request r within its plane, or -1 when
 * its table index or page id is out of range (as for whole rows). */
static int64_t head_offset(const head_side* s, int64_t Db, int64_t r, int64_t t, int64_t h)
{
    int64_t k = t / s->page_size;              /* the index checked as in page_of */
    if (s->pg_off[r] < -k || s->pg_off[r] >= s->num_ids - k) return -1;
    int64_t idx = s->pg_off[r] + k;
    int64_t page = (int64_t)s->ids[idx];
    if (page < 0 || page >= s->num_pages) return -1;
    int64_t row = t % s->page_size;
    if (s->hnd) return page * s->page_size * s->stride + (h * s->page_size + row) * Db;
    return (page * s->page_size + row) * s->stride + h * Db;
}

static void* run_heads(void* arg)
{
    head_job* j = (head_job*)arg;
    int64_t skipped = 0;
    for (int64_t pair = j->first_pair; pair < j->last_pair; ++pair) {
        int64_t r = pair / j->Q;
        int64_t q = pair % j->Q;
        int64_t n = j->tok_off[r + 1] - j->tok_off[r];
        for (int64_t t = 0; t < n; ++t) {
            if (head_offset(&j->src, j->Db, r, t, j->src.h0) < 0 ||
                head_offset(&j->dst, j->Db, r, t, j->dst.h0) < 0) {
                ++skipped;
                continue;
            }
            for (int32_t k = 0; k < j->nh; ++k) {
                int64_t so = head_offset(&j->src, j->Db, r, t, j->src.h0 + k);
                int64_t d = head_offset(&j->dst, j->Db, r, t, j->dst.h0 + k);
                memcpy(j->dst.planes[q] + d, j->src.planes[q] + so, (size_t)j->Db);
            }
        }
    }
    j->skipped = skipped;
    return NULL;
}

int64_t oracle_gather_scatter_heads(int32_t Q, int32_t nh, int64_t Db,
                                    uint8_t* const* src_planes, int64_t src_stride,
                                    int32_t src_page_size, int64_t src_num_pages,
                                    const int64_t* src_pg_off, const int32_t* src_ids,
                                    int64_t src_num_ids,
                                    int32_t src_H, int32_t src_h0, int32_t src_hnd,
                                    int32_t num_reqs, const int64_t* tok_off,
                                    uint8_t* const* dst_planes, int64_t dst_stride,
                                    int32_t dst_page_size, int64_t dst_num_pages,
                                    const int64_t* dst_pg_off, const int32_t* dst_ids,
                                    int64_t dst_num_ids,
                                    int32_t dst_H, int32_t dst_h0, int32_t dst_hnd,
                                    int nthreads)
{
    head_job proto;
    memset(&proto, 0, sizeof proto);
    proto.Q = Q; proto.nh = nh; proto.Db = Db; proto.num_reqs = num_reqs; proto.tok_off = tok_off;
    head_side s = {src_planes, src_stride, src_page_size, src_num_pages, src_pg_off, src_ids,
                   src_num_ids, src_H, src_h0, src_hnd};
    head_side d = {dst_planes, dst_stride, dst_page_size, dst_num_pages, dst_pg_off, dst_ids,
                   dst_num_ids, dst_H, dst_h0, dst_hnd};
    proto.src = s;
    proto.dst = d;
    int64_t pairs = (int64_t)num_reqs * Q;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (pairs < nthreads) nthreads = pairs > 0 ? (int)pairs : 1;
    head_job jobs[256];
    pthread_t tids[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].first_pair = pairs * i / nthreads;
        jobs[i].last_pair = pairs * (i + 1) / nthreads;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&tids[i], NULL, run_heads, &jobs[i]) == 0;
    run_heads(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(tids[i], NULL);
        else run_heads(&jobs[i]);
    }
    int64_t total = 0;
    for (int i = 0; i < nthreads; ++i) total += jobs[i].skipped;
    return total;
}

/* ------------------------------------------------------------- permutes -- */

typedef struct {
    int rebuild;
    int32_t H;
    int64_t Db;              /* head_dim * element size */
    int64_t s_cap, seq;
    uint8_t* const* hf;      /* [Q] planes, each [1][H][s_cap][D] */
    uint8_t* flat;           /* [Q][seq][H][D] */
    int32_t q0, q1;
} perm_job;

static void* run_perm(void* arg)
{
    perm_job* j = (perm_job*)arg;
    for (int32_t q = j->q0; q < j->q1; ++q)
        for (int64_t s = 0; s < j->seq; ++s)
            for (int32_t h = 0; h < j->H; ++h) {
                uint8_t* hf_row = j->hf[q] + ((int64_t)h * j->s_cap + s) * j->Db;
                uint8_t* flat_row = j->flat + (((int64_t)q * j->seq + s) * j->H + h) * j->Db;
                if (j->rebuild) memcpy(hf_row, flat_row, (size_t)j->Db);
                else memcpy(flat_row, hf_row, (size_t)j->Db);
            }
    return NULL;
}

static void run_perm_split(perm_job proto, int32_t Q, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (Q < nthreads) nthreads = Q > 0 ? Q : 1;
    perm_job jobs[256];
    pthread_t tids[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].q0 = (int32_t)((int64_t)Q * i / nthreads);
        jobs[i].q1 = (int32_t)((int64_t)Q * (i + 1) / nthreads);
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&tids[i], NULL, run_perm, &jobs[i]) == 0;
    run_perm(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(tids[i], NULL);
        else run_perm(&jobs[i]);
    }
}

/* Extract: out[q][s][h][:] <- hf[q][0][h][s][:] for s < seq. */
int64_t oracle_extract_permute(int32_t Q, int32_t H, int64_t Db,
                               uint8_t* const* hf_planes, int64_t s_cap, int64_t seq,
                               uint8_t* out, int nthreads)
{
    perm_job j;
    memset(&j, 0, sizeof j);
    j.rebuild = 0; j.H = H; j.Db = Db; j.s_cap = s_cap; j.seq = seq;
    j.hf = hf_planes; j.flat = out;
    run_perm_split(j, Q, nthreads);
    return 0;
}

/* Rebuild: hf[q][0][h][s][:] <- in[q][s][h][:] for s < seq; s >= seq untouched. */
int64_t oracle_rebuild_permute(int32_t Q, int32_t H, int64_t Db,
                               const uint8_t* in, int64_t seq,
                               uint8_t* const* hf_planes, int64_t s_cap, int nthreads)
{
    perm_job j;
    memset(&j, 0, sizeof j);
    j.rebuild = 1; j.H = H; j.Db = Db; j.s_cap = s_cap; j.seq = seq;
    j.hf = hf_planes; j.flat = (uint8_t*)in;
    run_perm_split(j, Q, nthreads);
    return 0;
}
