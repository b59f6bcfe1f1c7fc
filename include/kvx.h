/*
 * kvx.h -- C ABI of libkvx.so: paged KV-cache gather, scatter, pool-to-pool
 * gather-scatter and the HF [1, H, S, D] <-> [S, H, D] permutes, on one
 * MI355X (gfx950) GPU.
 *
 * Sources (the pages' titles and the sections each call follows):
 *   [budget]  "穷人版 PD 分离：在消费级显卡上把 TTS 推理拆成两半" (kilerd.me,
 *             pd-on-a-budget): "B300：让 P 直接写 D 的显存" (a kernel writes the
 *             scattered source rows straight into D's pages) and
 *             "5090：一个看得见所有卡的代理" (a token-paged pool leaves one
 *             request's KV in thousands of few-KB pieces; P gathers them into
 *             contiguous staging, D scatters them back into its pages).
 *   [mini]    "mini-infer系统实战-18-PD 解耦：把 Prefill 和 Decode 拆进两个进程之后
 *             发生了什么" (smarter.xin): "KV 序列化格式选择" (per-layer (k, v)
 *             tensors [seq, kv_heads, head_dim] extracted from and rebuilt
 *             into the HF [batch, heads, seq, dim] cache).
 *   [survey]  "PD分离调研：从推理阶段拆分到Mooncake的KVCache中心架构"
 *             (gentlecold.top): 6.1 (a batch of non-contiguous src/dst
 *             transfers submitted at once), 7.4 (per-layer cache base
 *             addresses and block length = tensor bytes / num_blocks), 7.6
 *             (P builds src/dst/length lists from block ids and writes D's
 *             KV blocks directly), 7.7 (P and D with different tensor-parallel
 *             sizes move the head ranges they share; head-major blocks).
 *   [distserve] "DistServe 完全拆解：拆开 Prefill 与 Decode，按 Goodput 调度大模型
 *             推理" (pinghaoyang.com.cn): "KV Cache 跨实例传输：省下重算，付出通信"
 *             (bytes per request = 2 x prompt length x layers x KV heads x
 *             head dim x element bytes).
 *
 * Conventions shared by every call
 * --------------------------------
 * Row.    One token of one plane: kv_heads * head_dim elements, R bytes.
 * Plane.  q = layer * num_kv + kv (kv = 0 for K, 1 for V); Q = num_layers *
 *         num_kv planes.  Each plane of a pool is an array of slots of R
 *         bytes: slot s of plane q starts at planes[q] + s * slot_stride
 *         (slot_stride = R for a layer-major [slots, H, D] tensor per plane,
 *         Q * R for a token-major pool).
 * Pages.  A pool holds num_pages pages of page_size consecutive slots.
 *         Token t of request r lives in page ids[pg_off[r] + t / page_size],
 *         at slot page * page_size + t % page_size.  page_size = 1 is the
 *         token-paged pool of [budget]; 16 is a vLLM-style block ([survey] 7.4).
 * Staging. Request r's rows start at byte tok_off[r] * Q * R; inside it the
 *         layout is [q][t][h][d]: the per-layer (k, v) [seq, H, D] tensors of
 *         [mini], concatenated plane by plane, then request by request.
 * Copy.   Every call is a bitwise copy of whole rows: dtype only fixes the
 *         element size; NaN payloads, -0 and subnormals are preserved.
 *
 * Asynchrony and ownership.  Every call validates its arguments on the host,
 * enqueues its kernel(s) on `stream` and returns without synchronising.  The
 * library allocates nothing, keeps no state between calls (apart from a
 * cached compute-unit count per device) and needs no memory registration: on
 * one GPU every device pointer is usable as is.  The caller owns every buffer
 * (pools, staging, tables, counter).  Host arrays (plane pointer lists, the
 * structs themselves) are read only during the call.  Device inputs must stay
 * alive and unmodified, and destination rows must not be read or reused,
 * until the stream has passed the call: completion of the stream (an event
 * or a synchronisation) is the only proof that every write has landed.
 *
 * Errors.  Argument errors return a nonzero kvx_status and enqueue nothing.
 * KVX_E_HIP means the launch itself was refused by the HIP runtime; faults
 * inside a kernel surface at the caller's next synchronisation, as for any
 * HIP kernel.  There is no fallback to a slower path: an unsupported case is
 * an error status.
 *
 * Page-table reads.  Token t of request r takes its page id from
 * page_ids[pg_off[r] + t / page_size]: a request's list is read from its
 * start onward, one entry per page of its tokens, and the data-movement
 * calls never read pg_off[r + 1], so a list shorter than ceil(n_r /
 * page_size) entries runs on into the entries after it (kvx_check_tables
 * reports such a list).
 *
 * Out-of-range rows.  A row whose page-table index pg_off[r] + t /
 * page_size falls outside [0, num_ids), or whose page id falls outside
 * [0, num_pages), is never dereferenced: it is skipped, its destination
 * bytes keep their prior contents, and (when `skipped` is not NULL) it is
 * added to *skipped with a device atomic.  A token of a pool-to-pool copy
 * that is out of range on either side is skipped in every plane.  No write
 * can land outside the destination pool or staging, whatever the tables
 * hold ([budget], failure-handling section: a late write landing in pages
 * that were already given to another request is the failure to rule out).
 *
 * Token offsets.  tok_off must follow its contract (kvx_reqs below).  The
 * calls cannot check it without reading device memory; KVX_VALIDATE=1 does,
 * and refuses a violation with KVX_E_SHAPE.  With a tok_off that breaks the
 * contract the kernels still address nothing outside the pools and the
 * staging (every staging row they form lies below total_tokens * Q * R
 * bytes, and pool rows are bounded as above), but which rows are copied is
 * then unspecified.
 *
 * Preconditions the data-movement calls do not check (they would need the
 * device tables on the host): within one call the destination rows are
 * pairwise distinct, and source and destination bytes do not overlap.  Under
 * them the result is unique and equals the row-by-row definition above.
 * kvx_check_tables and kvx_check_disjoint (below) check them on host copies
 * of the tables, as a debug aid.  With KVX_VALIDATE=1 in the environment
 * (read once per process) every data-movement call runs those checks itself
 * before enqueueing: it synchronizes its stream, copies its tables to the
 * host, and returns KVX_E_SHAPE for a tok_off that breaks its contract, or
 * KVX_E_DUPLICATE or KVX_E_OVERLAP for rows that violate the preconditions,
 * with nothing enqueued (out-of-range rows stay legal).  Debug only: it
 * cannot run on a stream under graph capture (KVX_E_HIP).  KVX_LOG=1 prints
 * each launch decision to stderr.
 */
#ifndef KVX_H
#define KVX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVX_ABI_VERSION 6

typedef enum kvx_status {
    KVX_OK = 0,
    KVX_E_NULL = 1,         /* a required pointer (struct, plane, table, buffer) is NULL */
    KVX_E_SHAPE = 2,        /* counts or sizes are negative, inconsistent or too small */
    KVX_E_ALIGN = 3,        /* a plane base, stride, buffer or row size is not a multiple of 16 B */
    KVX_E_DTYPE = 4,        /* unknown kvx_dtype code */
    KVX_E_RANGE = 5,        /* a size beyond what one call supports (see each limit below) */
    KVX_E_UNSUPPORTED = 6,  /* a valid request this build does not implement */
    KVX_E_HIP = 7,          /* the HIP runtime refused a launch or a device query */
    KVX_E_DUPLICATE = 8,    /* checkers: two written rows are the same row or overlap */
    KVX_E_OVERLAP = 9       /* kvx_check_disjoint: a written row overlaps a row the call reads */
} kvx_status;

typedef enum kvx_dtype {
    KVX_F16 = 1,            /* 2-byte elements */
    KVX_BF16 = 2,           /* 2-byte elements */
    KVX_FP8 = 3,            /* 1-byte elements */
    KVX_F32 = 4             /* 4-byte elements */
} kvx_dtype;

/* Row shape of a KV cache ([distserve] byte formula; [mini] tensor shapes).
 * R = kv_heads * head_dim * element size must be a multiple of 16 bytes and
 * at most 65536; Q = num_layers * num_kv. */
typedef struct kvx_layout {
    int32_t num_layers;     /* >= 1 */
    int32_t num_kv;         /* 2 for separate K and V planes, 1 for one latent plane per layer */
    int32_t kv_heads;       /* >= 1 */
    int32_t head_dim;       /* >= 1 */
    int32_t dtype;          /* a kvx_dtype */
} kvx_layout;

/* A paged pool ([survey] 7.4: per-layer cache base addresses, each cut into
 * num_blocks equal blocks).  planes is a HOST array of Q DEVICE pointers,
 * each 16-byte aligned and addressing at least
 * (num_pages * page_size - 1) * slot_stride + R bytes (NULL allowed for an
 * empty pool, num_pages = 0, whose rows are never dereferenced).  A pool
 * that is the source of kvx_gather or kvx_gather_scatter must hold at least
 * one slot when the batch has tokens (KVX_E_SHAPE otherwise): rows that are
 * skipped read the plane's first slot and discard it.  Planes may be
 * separate arrays (layer-major, slot_stride = R) or interleaved slot by slot
 * (token-major, slot_stride = Q * R, planes[q] = base + q * R); the result
 * is the same, and the kernels order their work to suit the layout.
 *
 * Row i of page p of plane q starts at planes[q] + p * page_stride +
 * i * slot_stride.  page_stride 0 means page_size * slot_stride (a page holds
 * one plane's rows only, so slot s = p * page_size + i is at s *
 * slot_stride).  A nonzero page_stride is the block length of a tensor whose
 * blocks hold several planes' pages ([survey] 7.4: block length = tensor
 * bytes / num_blocks), e.g. a per-layer [num_blocks][2][page_size][H][D]
 * tensor with planes[K] = base and planes[V] = base + page_size * R, or one
 * [num_blocks][layers][2][page_size][H][D] tensor: a multiple of 16, at least
 * (page_size - 1) * slot_stride + R (the pages of a plane do not overlap;
 * KVX_E_SHAPE otherwise), a multiple of slot_stride (KVX_E_UNSUPPORTED
 * otherwise), and not accepted by kvx_gather_scatter_heads
 * (KVX_E_UNSUPPORTED).
 *
 * Layout and speed (results never depend on it): HBM serves two rows of a
 * plane together when they lie a multiple of 32 KiB apart inside one
 * 128 KiB-aligned block.  Pools whose pages hold 64 KiB or more of a plane,
 * whose blocks hold a layer's K and V pages side by side (pages of 32 or
 * 64 KiB), or that are token-major, with plane bases aligned to 64 KiB,
 * let the kernels run such rows together and move 10-20% faster than pages
 * of scattered single rows. */
typedef struct kvx_pool {
    void* const* planes;
    int64_t num_pages;      /* >= 0 */
    int32_t page_size;      /* tokens per page, >= 1 */
    int64_t slot_stride;    /* bytes between consecutive rows of a page, >= R, multiple of 16 */
    int64_t page_stride;    /* bytes between consecutive pages of a plane; 0: page_size * slot_stride */
} kvx_pool;

/* A batch of requests: request r owns tokens [tok_off[r], tok_off[r+1]) of the
 * batch.  tok_off is a DEVICE array of num_reqs + 1 int64 values with
 * tok_off[0] = 0, non-decreasing, tok_off[num_reqs] = total_tokens (a host
 * copy of the last entry, used for sizing the launch).  Empty requests are
 * allowed.  With num_reqs == 1 the kernels take tok_off = {0, total_tokens}
 * from this contract and do not read it (KVX_VALIDATE=1 still checks it). */
typedef struct kvx_reqs {
    int32_t num_reqs;       /* >= 0 */
    int64_t total_tokens;   /* >= 0 */
    const int64_t* tok_off; /* DEVICE [num_reqs + 1] */
} kvx_reqs;

/* Where a batch's tokens live in one pool ([survey] 7.5/7.6: per-request
 * block id lists).  Request r's page ids start at page_ids[pg_off[r]], one
 * per page of its tokens (ceil(n_r / page_size) of them); how indices past
 * the list or outside page_ids are read is stated under "Page-table reads"
 * and "Out-of-range rows" above.  pg_off values may be any int64. */
typedef struct kvx_table {
    const int64_t* pg_off;   /* DEVICE [num_reqs + 1] */
    const int32_t* page_ids; /* DEVICE [num_ids] */
    int64_t num_ids;         /* host: length of page_ids (reads never go past it) */
} kvx_table;

/* Output flags of the calls that write a contiguous output (kvx_gather's
 * staging, the permutes' outputs).  By default such an output is written with
 * nontemporal stores, the faster choice when nothing on this GPU reads it
 * back soon (it is sent to another GPU or host, or consumed much later).
 * KVX_OUT_CACHED asks for ordinary stores instead, which leave what fits of
 * the output in the L2 and the 256 MiB Infinity Cache for a consumer on the
 * same GPU that runs right after (e.g. a rebuild of the staging a gather has
 * just written).  The bytes written are the same either way.  Any other bit
 * is refused with KVX_E_UNSUPPORTED. */
#define KVX_OUT_CACHED 1u

/* Gather ([budget] 5090 section; [survey] 6.1): copy every row of every
 * request, all Q planes, from pool `src` into contiguous staging laid out as
 * described above.  staging_bytes must be >= total_tokens * Q * R.  Staging
 * rows of skipped tokens keep their prior contents.  flags: 0 or
 * KVX_OUT_CACHED (above).  One launch for the whole batch (two or more only
 * when Q > 128). */
kvx_status kvx_gather(const kvx_layout* layout, const kvx_pool* src, const kvx_table* src_table,
                      const kvx_reqs* reqs, void* staging, int64_t staging_bytes,
                      unsigned long long* skipped, uint32_t flags, hipStream_t stream);

/* Scatter ([budget] 5090 section): the inverse of kvx_gather -- copy staging
 * rows into pool `dst` at the slots of dst_table.  Every destination byte
 * outside the written rows (other slots, the unused rows of a partly filled
 * last page) is left untouched. */
kvx_status kvx_scatter(const kvx_layout* layout, const void* staging, int64_t staging_bytes,
                       const kvx_reqs* reqs, const kvx_pool* dst, const kvx_table* dst_table,
                       unsigned long long* skipped, hipStream_t stream);

/* Gather-scatter ([budget] B300 section; [survey] 7.6): copy each row of pool
 * `src` at its src_table slot directly to pool `dst` at its dst_table slot,
 * with no staging.  Both tables index the same request batch; the two pools
 * may differ in page size and slot stride, not in layout. */
kvx_status kvx_gather_scatter(const kvx_layout* layout,
                              const kvx_pool* src, const kvx_table* src_table,
                              const kvx_reqs* reqs,
                              const kvx_pool* dst, const kvx_table* dst_table,
                              unsigned long long* skipped, hipStream_t stream);

/* Block layout of a page in a head-sliced copy ([survey] 7.7: for P and D
 * with different tensor-parallel sizes, non-MLA models keep each block
 * head-major, so that one head of one block is contiguous). */
typedef enum kvx_block_layout {
    KVX_NHD = 0,            /* page = [page_size][kv_heads][head_dim] (token-major) */
    KVX_HND = 1             /* page = [kv_heads][page_size][head_dim] (head-major) */
} kvx_block_layout;

/* Which heads of every token row a head-sliced copy reads or writes in one
 * pool.  With that pool's kvx_pool, slot_stride is the bytes of one token row
 * (>= kv_heads * head_dim * element size), so a page spans page_size *
 * slot_stride bytes; head h of token t of a page then starts at
 *   NHD: (page * page_size + t % page_size) * slot_stride + h * Db
 *   HND: page * page_size * slot_stride + (h * page_size + t % page_size) * Db
 * from the plane base, Db = head_dim * element size.  Each plane of a pool
 * used in a head-sliced copy must span whole pages: num_pages * page_size *
 * slot_stride bytes. */
typedef struct kvx_heads {
    int32_t kv_heads;       /* heads per token row in this pool (one TP shard's count) */
    int32_t head0;          /* first head of the slice; head0 + slice width <= kv_heads */
    int32_t block_layout;   /* a kvx_block_layout */
} kvx_heads;

/* Head-sliced gather-scatter ([survey] 7.7): when P and D shard the KV heads
 * over different tensor-parallel sizes, a P rank and a D rank move only the
 * heads they share -- a contiguous range starting at src_heads->head0 in the
 * source rows and at dst_heads->head0 in the destination rows.  For every
 * request, plane and token, layout->kv_heads heads (the slice width) are
 * copied, head by head, from pool `src` to pool `dst`; either side may use
 * NHD or HND blocks (so a whole-row slice also converts between the two).
 * A token whose page id is out of range on either side is skipped and
 * counted once.  Requires head_dim * element size to be a multiple of 16
 * bytes, and a source pool with at least one slot when total_tokens > 0
 * (rows that are not copied read the plane's first bytes; KVX_E_SHAPE
 * otherwise).  One launch (two or more only when Q > 128). */
kvx_status kvx_gather_scatter_heads(const kvx_layout* layout,
                                    const kvx_pool* src, const kvx_table* src_table,
                                    const kvx_heads* src_heads,
                                    const kvx_reqs* reqs,
                                    const kvx_pool* dst, const kvx_table* dst_table,
                                    const kvx_heads* dst_heads,
                                    unsigned long long* skipped, hipStream_t stream);

/* Extract permute ([mini]): for each plane q, hf_planes[q] is a DEVICE
 * [1][H][s_cap][D] tensor (batch 1, contiguous); write
 * out[q][s][h][:] = hf_planes[q][0][h][s][:] for s < seq_len.  out is a
 * contiguous DEVICE [Q][seq_len][H][D] buffer of out_bytes >= Q * seq_len * R
 * bytes.  Requires seq_len <= s_cap and head_dim * element size a multiple of
 * 16 bytes.  hf_planes is a HOST array of Q DEVICE pointers.  A pointer to an
 * empty buffer may be NULL: the planes when s_cap is 0, out when seq_len is
 * 0 (with seq_len 0 nothing is read or written). */
kvx_status kvx_extract_permute(const kvx_layout* layout, const void* const* hf_planes,
                               int64_t s_cap, int64_t seq_len,
                               void* out, int64_t out_bytes, uint32_t flags, hipStream_t stream);

/* Rebuild permute ([mini]): the inverse of extract --
 * hf_planes[q][0][h][s][:] = in[q][s][h][:] for s < seq_len; positions
 * s >= seq_len keep their prior contents.  flags (both permutes): 0 or
 * KVX_OUT_CACHED, for the output (out of extract, the HF planes of
 * rebuild). */
kvx_status kvx_rebuild_permute(const kvx_layout* layout, const void* in, int64_t in_bytes,
                               int64_t seq_len, void* const* hf_planes, int64_t s_cap,
                               uint32_t flags, hipStream_t stream);

/* Precondition checker (debug aid; not on the data path).  Takes HOST copies
 * of a batch's token CSR and of one pool's page table and checks what the
 * data-movement calls assume but cannot check without reading device
 * memory: tok_off starts at 0, never decreases and ends at total_tokens;
 * pg_off starts at >= 0, never decreases, stays within num_ids, and gives
 * every request at least ceil(n_r / page_size) page ids; every page id a
 * token uses is in [0, num_pages); and, when `as_destination` is nonzero,
 * no two tokens map to the same slot (the rows a scatter or gather-scatter
 * writes must be pairwise distinct; [budget]'s failure-handling section:
 * two writers landing in the same page is the failure to rule out).
 * Returns KVX_OK, KVX_E_SHAPE (inconsistent offsets), KVX_E_RANGE (a page
 * id out of range) or KVX_E_DUPLICATE; *bad_token (if not NULL) receives the
 * offending batch token, or -1.  Unlike the data-movement calls it
 * allocates host memory (one bit per slot for the duplicate test) and
 * reads only host memory. */
kvx_status kvx_check_tables(int32_t num_reqs, int64_t total_tokens, const int64_t* tok_off,
                            const int64_t* pg_off, const int32_t* page_ids, int64_t num_ids,
                            int64_t num_pages, int32_t page_size, int32_t as_destination,
                            int64_t* bad_token);

/* Overlap checker (debug aid; not on the data path).  For one kvx_gather,
 * kvx_scatter or kvx_gather_scatter call, described with HOST copies of its
 * token CSR (reqs->tok_off) and page tables (pg_off, page_ids), checks that
 * the rows the call writes are pairwise disjoint and that none of them
 * overlaps a row the call reads: the two preconditions under which the
 * result is unique.  A side is a pool (kvx_pool plus its kvx_table) or, when
 * both of that side's pointers are NULL, the staging buffer `staging` of
 * staging_bytes bytes (its row of plane q of token t of request r at
 * (tok_off[r] * Q + q * n_r + t) * R, as in kvx_gather).  Plane pointers and
 * `staging` are compared as addresses and never dereferenced, so DEVICE
 * pointers are fine here.  A token with an out-of-range page id on a pool
 * side is left out (the call skips it and touches neither of its rows).
 * Returns KVX_OK, KVX_E_DUPLICATE (two written rows share a byte),
 * KVX_E_OVERLAP (a written row shares a byte with a read row; checked only
 * when no written rows overlap), or an argument status: KVX_E_NULL,
 * KVX_E_SHAPE (inconsistent offsets, tables or staging too small),
 * KVX_E_UNSUPPORTED (both sides staging).  *bad_token (if not NULL) receives
 * one batch token whose written row is at fault, or -1.  Host cost: 24 bytes
 * and O(log) sorting work per row on each side (Q * total_tokens rows). */
kvx_status kvx_check_disjoint(const kvx_layout* layout, const kvx_reqs* reqs,
                              const kvx_pool* src, const kvx_table* src_table,
                              const kvx_pool* dst, const kvx_table* dst_table,
                              const void* staging, int64_t staging_bytes,
                              int64_t* bad_token);

/* Static string naming a status code (never NULL; "unknown kvx_status" for a
 * code outside kvx_status).  Takes a plain int32_t so that any code a caller
 * holds, valid or not, is a well-defined argument. */
const char* kvx_status_str(int32_t status);

/* KVX_ABI_VERSION of the built library. */
int32_t kvx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVX_H */
