/*
 * top_selected_attention.h -- C ABI of the MI355X (gfx950) library for
 * attention restricted to selected key blocks.
 *
 * Three front-ends share one engine:
 *   - block-sparse attention (BSA): a BlockSparseMask names, per Q block, the
 *     KV blocks it attends to ("aclnnBlockSparseAttentionGrad", function
 *     description and formula section);
 *   - NSA selected attention: per (token, KV head) topk_indices name the
 *     selected key blocks ("aclnnNsaSelectedAttention", formulas section);
 *   - sparse flash attention (SFA) decode over a paged, shared KV cache with
 *     per-token top-k positions ("aclnnSparseFlashAttention", formulas and
 *     constraints sections; "SparseAttnSharedkvMetadata", parameter list).
 *
 * Calling pattern (the two-phase pattern of the CANN operator pages, "calls"
 * section of each): first XXX_workspace_size(args, &bytes) validates the
 * arguments on the host -- it never touches the device and never reads device
 * memory -- and returns the workspace size; then XXX(args, ws, ws_bytes,
 * stream) re-validates and enqueues the kernels on `stream`.
 *
 * Ownership: the caller owns every buffer, including the workspace.  The
 * library never allocates or frees device memory and keeps no device state
 * besides its loaded code objects (which hold the fixed scratch array of
 * sfa_paged_fwd_noalloc); calls other than that one are reentrant.  Device pointers are
 * borrowed until the work enqueued on `stream` completes.  Host pointers
 * (marked HOST) are read during the call only.
 *
 * Pointers marked DEVICE must be device memory of the current HIP device.
 * All tensors are dense and contiguous in the stated layout.  `stream` is a
 * hipStream_t (NULL = the null stream).  The kernels move rows in 16-byte
 * pieces: the workspace and the DEVICE pointers of q, k, v, out, dout, dq,
 * dk, dv, block_mask, q_rope and the key caches must be 16-byte aligned
 * (fresh allocations are); a misaligned tensor gives TSA_ERR_INVALID, a
 * misaligned workspace TSA_ERR_WORKSPACE.
 *
 * Every args struct ends with reuse_lists, n_events and events.  Stages
 * that can be timed, per entry point: bsa_fwd 0 = lists, 1 = attention;
 * bsa_bwd 0 = lists, 1 = dQ (with softmax_grad), 2 = dK/dV (the kernel), 3 = the
 * ordered reduction of the fp32 partials of split KV tiles; nsa_select_fwd
 * 0 = lists, 1 = attention; nsa_select_bwd 0 = lists, 1 = dQ, 2 = dK/dV
 * fp32 partials (segment table + partial kernel), 3 = their reduction;
 * sfa_paged_fwd 0 = split attention, 1 = split combine.  A stage that a call
 * skips records both of its events back to back.
 *
 * Errors: every function returns a tsa_status.  No exceptions cross the ABI
 * and nothing calls exit().  The CANN pages' own error-code tables were lost,
 * so the values below are this library's.
 */
#ifndef TOP_SELECTED_ATTENTION_H
#define TOP_SELECTED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define TSA_API __attribute__((visibility("default")))
#else
#define TSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TSA_OK = 0,
  TSA_ERR_NULL = 1,          /* a required pointer is NULL */
  TSA_ERR_INVALID = 2,       /* a value or shape violates a documented constraint */
  TSA_ERR_UNSUPPORTED = 3,   /* valid for the operator, not built in this library */
  TSA_ERR_WORKSPACE = 4,     /* workspace NULL, smaller than XXX_workspace_size or
                                not 16-byte aligned */
  TSA_ERR_HIP = 5,           /* a HIP launch or runtime call failed */
  TSA_ERR_DATA = 6,          /* validate = 1 found bad data (ids out of range) */
  TSA_ERR_SCRATCH = 7        /* a no-allocation call needs more than its fixed scratch */
} tsa_status;

enum { TSA_BF16 = 0, TSA_FP16 = 1 };
enum { TSA_LAYOUT_BNSD = 0, TSA_LAYOUT_TND = 1, TSA_LAYOUT_BSND = 2 };

/* Text for a status code (static storage, never NULL). */
TSA_API const char* tsa_status_string(int status);

/* sizeof of each argument struct, for binding checks: which = 0 bsa_fwd,
 * 1 bsa_bwd, 2 nsa_select_fwd, 3 nsa_select_bwd, 4 sfa_paged_fwd,
 * 5 sfa_sharedkv_fwd, 6 floyd_fwd, 7 floyd_bwd; returns 0 for an unknown
 * value. */
TSA_API size_t tsa_args_sizeof(int which);

/* ------------------------------------------------------------------------
 * Block-sparse attention.
 *
 * Forward ("aclnnBlockSparseAttentionGrad", formula section):
 *   Out = Softmax(Mask(scale * Q * K_sparse^T, atten_mask)) * V_sparse,
 * where K_sparse/V_sparse of a Q block are the rows of the KV blocks its mask
 * row selects.  Also writes LSE = row max + ln(row sum of exp), fp32 (natural
 * log), which the backward uses.
 *
 * Layouts (the page's layout section lists TND and BNSD for qInputLayout
 * and kvInputLayout; its constraints build only BNSD, both are built here,
 * with q and k/v in the same layout, else TSA_ERR_UNSUPPORTED):
 *   BNSD: q [B, N1, Sq, D], k [B, N2, Skv, D], v [B, N2, Skv, D], out like q,
 *     lse fp32 [B, N1, Sq].
 *   TND (varlen): q [T, N1, D], k [Tk, N2, D], v [Tk, N2, D], out like q,
 *     lse fp32 [T, N1]; cu_seqlens_q / cu_seqlens_kv are HOST int32 [B+1]
 *     prefix sums from 0 (T = cu_seqlens_q[B], Tk = cu_seqlens_kv[B]; the
 *     layout section makes the sequence lengths mandatory with TND).  Sq and
 *     Skv are then the longest query / key sequence: they size the mask, and
 *     each sequence's own length bounds its rows (mask entries of blocks past
 *     a sequence's end are ignored).  Causal positions are within a sequence.
 *   D must be 128 (constraints section: headdim=128).  N1 % N2 == 0
 *   (constraints section); query head n1 reads KV head n1/(N1/N2).
 * block_mask: u8 DEVICE [B, N1, ceil(Sq/block_q), ceil(Skv/block_kv)],
 *   non-zero = the Q block attends to that KV block (blockShapeX = block_q
 *   rows, blockShapeY = block_kv keys; function description).  Tail blocks of
 *   a ragged Sq / Skv are partial.
 * sparse_mode: 0 = the selected blocks in full; 2 = additionally causal,
 *   key position j <= query position i (top-left aligned).
 * atten_mask (optional; the formula's Mask operand, whose format the page
 *   does not give): u8 DEVICE, element (b, n1, i, j) at
 *   atten_mask[b*atten_mask_stride_b + n1*atten_mask_stride_n + i*Skv + j]
 *   for query position i < Sq and key position j < Skv (within the sequence
 *   for TND); non-zero = that score is excluded, zero = kept.  Strides are in
 *   elements, >= 0 (0 = one plane shared by every batch entry / head), else
 *   TSA_ERR_INVALID; the caller guarantees every addressed element is in its
 *   allocation.  It only excludes entries of the selected blocks and adds to
 *   the causal exclusions of sparse_mode 2; a row left with no key gets
 *   Out = 0 and LSE = -inf.  NULL = no element mask (strides ignored).
 * scale: finite and > 0.
 * block_q, block_kv: 1..65536 (any size; partial tiles are masked).
 * A Q block that selects nothing gets Out = 0 and LSE = -inf.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;            /* TSA_BF16 or TSA_FP16 (q, k, v, out, dout, dq, dk, dv) */
  int32_t q_layout;         /* TSA_LAYOUT_BNSD or TSA_LAYOUT_TND */
  int32_t kv_layout;        /* the same as q_layout */
  int32_t B, N1, N2, Sq, Skv, D;
  int32_t block_q, block_kv;
  int32_t sparse_mode;      /* 0 or 2 */
  float scale;              /* > 0, typically 1/sqrt(D) */
  int32_t validate;         /* reserved for BSA (masks cannot hold bad data); 0 */
  const uint8_t* block_mask;/* DEVICE */
  const void* q;            /* DEVICE */
  const void* k;            /* DEVICE */
  const void* v;            /* DEVICE */
  void* out;                /* DEVICE, written */
  float* lse;               /* DEVICE, written */
  int32_t reuse_lists;      /* 0: build the forward and reverse lists in the workspace;
                               1: they are there from an earlier bsa_fwd / bsa_bwd call with
                               the same mask and shapes on this workspace; skip building them;
                               other values: TSA_ERR_INVALID */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t: events[2i] / [2i+1] are
                               recorded on `stream` before / after stage i (see each entry) */
  const int32_t* cu_seqlens_q;  /* TND only: HOST [B+1] (ignored for BNSD) */
  const int32_t* cu_seqlens_kv; /* TND only: HOST [B+1] */
  const uint8_t* atten_mask;    /* DEVICE or NULL: element exclusions (see above) */
  int64_t atten_mask_stride_b;  /* elements between batch entries' [Sq, Skv] planes; 0 = shared */
  int64_t atten_mask_stride_n;  /* elements between query heads' planes; 0 = shared */
} bsa_fwd_args;

TSA_API int bsa_fwd_workspace_size(const bsa_fwd_args* args, size_t* bytes);
TSA_API int bsa_fwd(const bsa_fwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* Backward ("aclnnBlockSparseAttentionGrad", formula section):
 *   softmax_grad = rowsum(dOut * Out)   (the page's softmaxGrad(dOut, Out))
 *   dP = dOut V^T,  dS = P * (dP - softmax_grad),  dV = P^T dOut,
 *   dQ = (dS K) scale,  dK = (dS^T Q) scale,
 * over the selected blocks only; P is recomputed from Q, K and the forward's
 * LSE.  dK/dV of a KV head sum over its N1/N2 query heads and every Q block
 * that selected the row; rows nobody selects get 0.  Deterministic: no atomics,
 * a fixed summation order, bit-identical results across runs.
 * Same shape fields as the forward; out/dout like q, lse from bsa_fwd.
 * dq like q, dk/dv like k/v (all written in full). */
typedef struct {
  int32_t dtype;
  int32_t q_layout;
  int32_t kv_layout;
  int32_t B, N1, N2, Sq, Skv, D;
  int32_t block_q, block_kv;
  int32_t sparse_mode;
  float scale;
  int32_t validate;
  const uint8_t* block_mask;/* DEVICE */
  const void* q;            /* DEVICE */
  const void* k;            /* DEVICE */
  const void* v;            /* DEVICE */
  const void* out;          /* DEVICE, the forward output */
  const void* dout;         /* DEVICE */
  const float* lse;         /* DEVICE, the forward LSE */
  void* dq;                 /* DEVICE, written */
  void* dk;                 /* DEVICE, written */
  void* dv;                 /* DEVICE, written */
  int32_t reuse_lists;      /* 0: build the lists; 1: they are there from an earlier bsa_fwd /
                               bsa_bwd call with the same mask and shapes on this workspace
                               (bsa_fwd builds both directions); other values: TSA_ERR_INVALID */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t: events[2i] / [2i+1] are
                               recorded on `stream` before / after stage i (see each entry) */
  const int32_t* cu_seqlens_q;  /* TND only: HOST [B+1] (ignored for BNSD) */
  const int32_t* cu_seqlens_kv; /* TND only: HOST [B+1] */
  const uint8_t* atten_mask;    /* DEVICE or NULL: the forward's atten_mask */
  int64_t atten_mask_stride_b;
  int64_t atten_mask_stride_n;
} bsa_bwd_args;

TSA_API int bsa_bwd_workspace_size(const bsa_bwd_args* args, size_t* bytes);
TSA_API int bsa_bwd(const bsa_bwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* The selected-block lists of a BlockSparseMask, as the kernels use them
 * (exposed so they can be checked bit for bit).  Uses args->B, N1, N2, Sq,
 * Skv, block_q, block_kv and block_mask only.  With R = B*N1*QB rows and
 * C = B*N2*KB KV blocks (QB = ceil(Sq/block_q), KB = ceil(Skv/block_kv)):
 *   row_ptr int32 DEVICE [R+1]: CSR pointers, row (b, n1, qb) row-major;
 *   col     int32 DEVICE [R*KB]: ascending kb per row (first row_ptr[R] used);
 *   rev_ptr int32 DEVICE [C+1]: CSR pointers, row (b, n2, kb) row-major;
 *   rev     int32 DEVICE [R*KB]: per KV block, ascending ids g*QB + qb of the
 *           Q blocks of query heads n1 = n2*G + g that selected it.
 * Needs a workspace of bsa_compact_workspace_size bytes. */
TSA_API int bsa_compact_workspace_size(const bsa_fwd_args* args, size_t* bytes);
TSA_API int bsa_compact(const bsa_fwd_args* args, int32_t* row_ptr, int32_t* col, int32_t* rev_ptr,
                int32_t* rev, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * NSA selected attention ("aclnnNsaSelectedAttention").
 *
 * Forward (formulas section): selected_key/value = Gather(key/value,
 * topk_indices[i]) for 0 <= i < selected_block_count; attention_out =
 * Softmax(Mask(scale * query @ selected_key^T, atten_mask)) @ selected_value.
 * Backward: the chain of "aclnnBlockSparseAttentionGrad" (formula section)
 * applied to the gathered keys, each gathered row's gradient added back to
 * its source row (deterministic, no atomics).
 *
 * Layout TND only (constraints section): q [T, N1, D], k [Tk, N2, D],
 * v [Tk, N2, Dv], out [T, N1, Dv], lse fp32 [T, N1].  Dv = 128 and D = 128
 *   or 192 (the constraints section fixes the query/key and the value head
 *   dims to two values its extraction lost; read as 192 and 128, and the
 *   equal pair 128 / 128 is built too); other values: TSA_ERR_UNSUPPORTED.
 * cu_seqlens_q / cu_seqlens_kv: HOST int32 [B+1] prefix sums starting at 0
 *   ("SparseAttnSharedkvMetadata", parameter list: cu_seqlens are B+1 prefix
 *   sums); cu_seqlens_q[B] == T, cu_seqlens_kv[B] == Tk.
 * topk: int32 DEVICE [T, N2, sbc], block ids counted in units of sbs from the
 *   start of the token's own sequence; a listed id counts once per listing.
 * sbs (selected_block_size): multiple of 16, at most 128 (constraints).
 * sbc (selected_block_count): 1..128, sbs*sbc <= 8192 (constraints).
 * Every KV sequence length is >= sbs*sbc and a multiple of sbs (constraints).
 * N1 % N2 == 0, G = N1/N2 <= 32.
 * sparse_mode: 0 = no mask; 2 = causal, key j <= query position i within
 *   the sequence; blocks wholly after the query are skipped.
 * validate = 1: one extra device pass checks that every id is in range
 *   (0 <= id < ceil(Skv_b/sbs)) and synchronises `stream`; TSA_ERR_DATA if
 *   not.  With validate = 0 out-of-range ids are skipped.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;
  int32_t layout;           /* TSA_LAYOUT_TND */
  int32_t B;                /* number of sequences */
  int32_t T, Tk;            /* total query / key tokens */
  int32_t N1, N2, D, Dv;
  const int32_t* cu_seqlens_q;   /* HOST [B+1] */
  const int32_t* cu_seqlens_kv;  /* HOST [B+1] */
  int32_t sbs, sbc;
  int32_t sparse_mode;      /* 0 or 2 */
  float scale;              /* finite, > 0 */
  int32_t validate;
  const int32_t* topk;      /* DEVICE [T, N2, sbc] */
  const void* q;            /* DEVICE */
  const void* k;            /* DEVICE */
  const void* v;            /* DEVICE */
  void* out;                /* DEVICE, written */
  float* lse;               /* DEVICE, written */
  int32_t reuse_lists;      /* 0: build the per-row lists (and, for head groups of up to 16
                               with 128-dim heads, the token-group chunk lists the forward and
                               dQ kernels walk; the reverse lists are left to the backward);
                               1: they are there from an earlier call with the same indices on
                               this workspace; other values: TSA_ERR_INVALID */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t: events[2i] / [2i+1] are
                               recorded on `stream` before / after stage i (see each entry) */
} nsa_select_fwd_args;

TSA_API int nsa_select_fwd_workspace_size(const nsa_select_fwd_args* args, size_t* bytes);
TSA_API int nsa_select_fwd(const nsa_select_fwd_args* args, void* workspace, size_t workspace_bytes,
                   void* stream);

typedef struct {
  int32_t dtype;
  int32_t layout;
  int32_t B;
  int32_t T, Tk;
  int32_t N1, N2, D, Dv;
  const int32_t* cu_seqlens_q;   /* HOST [B+1] */
  const int32_t* cu_seqlens_kv;  /* HOST [B+1] */
  int32_t sbs, sbc;
  int32_t sparse_mode;
  float scale;
  int32_t validate;
  const int32_t* topk;      /* DEVICE */
  const void* q;            /* DEVICE */
  const void* k;            /* DEVICE */
  const void* v;            /* DEVICE */
  const void* out;          /* DEVICE, forward output */
  const void* dout;         /* DEVICE */
  const float* lse;         /* DEVICE, forward LSE */
  void* dq;                 /* DEVICE, written [T, N1, D] */
  void* dk;                 /* DEVICE, written [Tk, N2, D] */
  void* dv;                 /* DEVICE, written [Tk, N2, Dv] */
  int32_t reuse_lists;      /* 0: build per-row and reverse lists; 1: both are there from an
                               earlier nsa_select_bwd call with the same indices on this
                               workspace; 2: the per-row (and token-group) lists are there
                               from an earlier nsa_select_fwd call with the same indices and
                               cu_seqlens on this workspace (its size being this call's):
                               build only the reverse
                               lists; other values: TSA_ERR_INVALID */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t: events[2i] / [2i+1] are
                               recorded on `stream` before / after stage i (see each entry) */
} nsa_select_bwd_args;

TSA_API int nsa_select_bwd_workspace_size(const nsa_select_bwd_args* args, size_t* bytes);
TSA_API int nsa_select_bwd(const nsa_select_bwd_args* args, void* workspace, size_t workspace_bytes,
                   void* stream);

/* The lists of topk_indices, as the kernels use them.  Uses the shape fields,
 * cu_seqlens, sbs, sbc, sparse_mode and topk of args; q, k, v, out and lse
 * are not read and may be NULL.  With R = T*N2 rows and
 * NB = sum_b ceil(Skv_b/sbs) blocks:
 *   row_ptr int32 DEVICE [R+1]; col int32 DEVICE [R*sbc]: per (t, n2) the
 *     block ids sorted ascending (mode 2: blocks wholly after t dropped);
 *   rev_ptr int32 DEVICE [N2*NB+1]; rev int32 DEVICE [R*sbc]: per (n2, global
 *     block) the ascending token ids whose row holds it.
 * nsa_compact_blocks_total() gives NB. */
TSA_API int nsa_compact_blocks_total(const nsa_select_fwd_args* args, int32_t* blocks_total);
TSA_API int nsa_compact_workspace_size(const nsa_select_fwd_args* args, size_t* bytes);
TSA_API int nsa_compact(const nsa_select_fwd_args* args, int32_t* row_ptr, int32_t* col,
                int32_t* rev_ptr, int32_t* rev, void* workspace, size_t workspace_bytes,
                void* stream);

/* ------------------------------------------------------------------------
 * Sparse flash attention, paged shared-KV decode ("aclnnSparseFlashAttention").
 *
 * Formulas section: softmax(Q K~^T / sqrt(d_k)) V~ over the selected keys;
 * a score is scale * (q . k + q_rope . k_rope).  Constraints section:
 * D = 512 for query/key/value, Dr = 64 for the rope parts, N1 in {1, 2, 4,
 * ..., 128}, page block_size a multiple of 16 and at most 1024, one dtype
 * for query/key/value.  "SparseAttnSharedkvMetadata" parameter list: one KV
 * head, PA_ND paged KV, seqused_kv = active KV length per batch, mask mode
 * 3 = rightDownCausal.
 *
 * q [B, Sq, N1, D], q_rope [B, Sq, N1, Dr] (BSND), or with q_layout TND
 *   ("SparseAttnSharedkvMetadata": layout_q BSND or TND, cu_seqlens_q the
 *   B+1 prefix sums of each entry's query tokens) q [T, N1, D], q_rope
 *   [T, N1, Dr], rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 belonging to
 *   entry b; Sq is then ignored and entry b's Sq_b = cu[b+1] - cu[b] sets
 *   its causal offset; topk_indices [T, N2, topk], out [T, N1, Dv], lse
 *   [T, N1].
 * key_cache [num_pages, page_size, N2, D], key_rope_cache [num_pages,
 *   page_size, N2, Dr], value_cache [num_pages, page_size, N2, Dv] (PA_ND,
 *   paged like the key cache through the same block table); value_cache may
 *   equal key_cache (shared KV: V is the key row, gathered once) or be a
 *   cache of its own (its rows are gathered beside the key rows).
 * block_table int32 DEVICE [B, max_pages]: physical page of logical page p.
 * kv_lens int32 DEVICE [B]: active KV tokens of each sequence.
 * topk_indices int32 DEVICE [B, Sq, N2, topk]: selected sparse-block ids
 *   (token positions when sparse_block_size == 1); -1 = empty slot.
 * sparse_block_size: divides page_size (reading of the constraint that ties
 *   it to block_size: a selected block never straddles a page); 1..page_size.
 * sparse_mode: 0 = no mask; 3 = rightDownCausal (token s of Sq sits at
 *   position kv_len - Sq + s, Sq_b for TND; later keys are masked).
 * out [B, Sq, N1, Dv]; lse fp32 [B, Sq, N1] (may be NULL).
 * validate = 1: checks ids, kv_lens and page ids on the device, synchronises
 *   `stream`, TSA_ERR_DATA on a bad value; with validate = 0 positions at or
 *   beyond kv_len are skipped.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;
  int32_t q_layout;         /* TSA_LAYOUT_BSND or TSA_LAYOUT_TND */
  int32_t B, Sq, N1, N2, D, Dr, Dv;
  int32_t num_pages, page_size, max_pages;
  int32_t topk;
  int32_t sparse_block_size;
  int32_t sparse_mode;      /* 0 or 3 */
  float scale;              /* finite, > 0 */
  int32_t validate;
  const void* q;            /* DEVICE */
  const void* q_rope;       /* DEVICE */
  const void* key_cache;    /* DEVICE */
  const void* key_rope_cache;/* DEVICE */
  const void* value_cache;  /* DEVICE */
  const int32_t* block_table;   /* DEVICE */
  const int32_t* kv_lens;       /* DEVICE */
  const int32_t* topk_indices;  /* DEVICE */
  void* out;                /* DEVICE, written */
  float* lse;               /* DEVICE, written, or NULL */
  int32_t reuse_lists;      /* unused (no lists); keep 0 */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t: events[2i] / [2i+1] are
                               recorded on `stream` before / after stage i (see each entry) */
  int32_t T;                    /* TND: total query tokens (== cu_seqlens_q[B]) */
  const int32_t* cu_seqlens_q;  /* TND: HOST [B+1] prefix sums from 0 (ignored for BSND) */
} sfa_paged_fwd_args;

TSA_API int sfa_paged_fwd_workspace_size(const sfa_paged_fwd_args* args, size_t* bytes);
TSA_API int sfa_paged_fwd(const sfa_paged_fwd_args* args, void* workspace, size_t workspace_bytes,
                  void* stream);

/* sfa_paged_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * it takes its workspace from a fixed array of the library's own, one per
 * GPU, that lives until the process ends, and calls no hipMalloc, hipFree
 * or other allocating routine.  The caller still owns q, the caches, the
 * tables, out and lse.  Same arguments, validation and results as
 * sfa_paged_fwd; a call whose workspace would exceed
 * sfa_paged_fwd_noalloc_max_bytes() (64 MiB: e.g. 128 decode tokens of 64
 * heads with 2 splits need 32 MiB) returns TSA_ERR_SCRATCH before any launch.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  The array keeps the last call's partial results; nothing in it
 * has to start at zero. */
TSA_API size_t sfa_paged_fwd_noalloc_max_bytes(void);
TSA_API int sfa_paged_fwd_noalloc(const sfa_paged_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Shared-KV two-branch sparse decode ("SparseAttnSharedkvMetadata",
 * parameter list; scores and values as in "aclnnSparseFlashAttention").
 *
 * Each decode token attends, in one softmax, to
 *   - the original KV (ori_kv, has_ori_kv = 1) under mask mode 4, a band of
 *     ori_win_left past and ori_win_right future positions around its own
 *     position p = seqused_kv[b] - Sq_b + s, clipped to [0, seqused_kv[b]);
 *   - cmp_topk selected entries of the compressed KV (cmp_kv, has_cmp_kv =
 *     1; the original compressed by cmp_ratio, so entry b holds
 *     seqused_kv[b] / cmp_ratio entries) under mask mode 3, rightDownCausal:
 *     compressed id c is kept iff c <= cmp_len - Sq_b + s.
 * score = scale * (q . k + q_rope . k_rope); the value is the key's 512-wide
 * row (shared KV); one KV head (num_heads_kv = 1).  Both caches are PA_ND:
 * key cache [pages, page_size, 1, 512], rope cache [pages, page_size, 1, 64],
 * block table int32 [B, max_pages] (DEVICE).
 * q [B, Sq, N1, 512], q_rope [B, Sq, N1, 64] (BSND) or [T, N1, ...] (TND
 * with HOST cu_seqlens_q [B+1]); cmp_topk_indices int32 DEVICE [tokens, 1,
 * cmp_topk] (-1 = empty); out like q with 512 columns; lse fp32 [tokens, N1]
 * (may be NULL).  A token with no kept key gets Out = 0, LSE = -inf.
 *
 * Task list (the metadata page's per-core list of tasks with their start
 * and end points): sfa_sharedkv_metadata writes, into a caller buffer of
 * sfa_sharedkv_metadata_size bytes, each token's batch entry and its slots
 * (the band padded to a multiple of 32, then the top-k slots) cut into
 * per-workgroup slot ranges of near-equal kept-key weight.  sfa_sharedkv_fwd
 * takes such a list in `tasks` (DEVICE) and then uploads and computes
 * nothing before the attention; with tasks == NULL it makes the list itself
 * in its workspace first.  A list made for the same shapes, cu_seqlens_q,
 * band and cmp_topk is valid for any ids and seqused_kv (those only steer
 * the balance), so one list can serve every layer of a decode step.  The
 * split kernel takes its range from the list and the combine kernel merges
 * the ranges by LSE.  Stages: 0 = task list (recorded back to back when
 * `tasks` is given), 1 = split attention, 2 = combine.
 * Constraints: N1 a power of two <= 128; D 512, Dr 64; page sizes multiples
 * of 16 <= 1024; cmp_ratio 4 or 128 (the parameter list's range);
 * ori_win_left, ori_win_right >= 0 with their band <= 4096 slots;
 * cmp_topk >= 1; at least one branch; scale finite and > 0.  Ids at or past
 * the compressed length are skipped.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;
  int32_t q_layout;             /* TSA_LAYOUT_BSND or TSA_LAYOUT_TND */
  int32_t B, Sq, T, N1, N2, D, Dr;
  float scale;
  const void* q;                /* DEVICE */
  const void* q_rope;           /* DEVICE */
  const int32_t* cu_seqlens_q;  /* TND: HOST [B+1] */
  const int32_t* seqused_kv;    /* DEVICE [B]: original KV tokens of each entry */
  int32_t has_ori_kv, has_cmp_kv;
  int32_t ori_win_left, ori_win_right;   /* 127, 0 */
  int32_t ori_num_pages, ori_page_size, ori_max_pages;
  const void* ori_key_cache;             /* DEVICE */
  const void* ori_key_rope_cache;        /* DEVICE */
  const int32_t* ori_block_table;        /* DEVICE */
  int32_t cmp_ratio;                     /* 4 or 128 */
  int32_t cmp_topk;
  int32_t cmp_num_pages, cmp_page_size, cmp_max_pages;
  const void* cmp_key_cache;             /* DEVICE */
  const void* cmp_key_rope_cache;        /* DEVICE */
  const int32_t* cmp_block_table;        /* DEVICE */
  const int32_t* cmp_topk_indices;       /* DEVICE */
  void* out;                    /* DEVICE, written */
  float* lse;                   /* DEVICE, written, or NULL */
  const void* tasks;            /* DEVICE task list from sfa_sharedkv_metadata (16-byte
                                   aligned, else TSA_ERR_INVALID), or NULL */
  int32_t reuse_lists;          /* unused; keep 0 */
  int32_t n_events;             /* number of stages to time (0 = off) */
  void* const* events;          /* HOST array of 2*n_events hipEvent_t (see above) */
} sfa_sharedkv_fwd_args;

/* Bytes of the task list of these arguments (validates them like the
 * forward; `tasks` is not read). */
TSA_API int sfa_sharedkv_metadata_size(const sfa_sharedkv_fwd_args* args, size_t* bytes);
/* Writes the task list into `tasks` (DEVICE, 16-byte aligned, at least the
 * size above; owned by the caller), enqueued on `stream`; reads cu_seqlens_q
 * (HOST, TND), seqused_kv and cmp_topk_indices (DEVICE).  NULL or too small:
 * TSA_ERR_WORKSPACE; misaligned: TSA_ERR_INVALID. */
TSA_API int sfa_sharedkv_metadata(const sfa_sharedkv_fwd_args* args, void* tasks,
                                  size_t tasks_bytes, void* stream);
TSA_API int sfa_sharedkv_fwd_workspace_size(const sfa_sharedkv_fwd_args* args, size_t* bytes);
TSA_API int sfa_sharedkv_fwd(const sfa_sharedkv_fwd_args* args, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FloydAttention ("aclnnFusedFloydAttentionGrad", function description and
 * formula section): the query keeps two sequence axes, and the scores of
 * query row (n, m) against key k add two products, each batched over one of
 * those axes:
 *   S = scale * (Q K1^T + Q K2^T),  P = Softmax over k (S),  Y = P V1 + P V2;
 * backward: dP = dY V1^T + dY V2^T, dS = P * (dP - rowsum(dY * Y)),
 *   dV1 = P^T dY, dV2 = P^T dY, dQ = (dS K1 + dS K2) scale,
 *   dK1 = dS^T Q scale, dK2 = dS^T Q scale.
 * Layouts (the page's shape table is lost; read from its constraints: axes
 * 0, 2 and 4 of query and key1 agree, key1/value1 and key2/value2 share
 * shapes, and the second pair is batched over the query's other sequence
 * axis): q [B, H, N, M, D]; k1, v1 [B, H, N, K, D]; k2, v2 [B, H, M, K, D];
 * out like q; lse fp32 [B, H, N, M] (one natural-log LSE per query row: the
 * page's softmaxMax / softmaxSum pair carries the same).
 * Constraints (shape constraints, read in this order): B in [1, 2048], H in
 * [1, 256], N a multiple of 16 in [16, 2^20], M and K multiples of 128 in
 * [128, 2^20], D in {32, 64, 128}; scale finite and > 0.  No atten_mask
 * (the page gives no layout for it).
 * Built from small operators (the page advises them once M x D or K x D is
 * large): strided batched MFMA GEMMs with the scores materialised in the
 * workspace (fp32 S and a 16-bit P, plus fp32 dP and a 16-bit dS in the
 * backward, B*H*N*M*K elements each, and an fp32 [B*H*N*M*D] accumulator).
 * Deterministic (no atomics).  Stages: forward 0 = scores, 1 = softmax,
 * 2 = P V1 + P V2; backward 0 = scores and dP, 1 = P and dS, 2 = dV1 / dV2,
 * 3 = dQ, 4 = dK1 / dK2.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;            /* TSA_BF16 or TSA_FP16 (every 16-bit tensor) */
  int32_t B, H, N, M, K, D;
  float scale;              /* finite, > 0; typically 1/sqrt(D) */
  const void* q;            /* DEVICE [B, H, N, M, D] */
  const void* k1;           /* DEVICE [B, H, N, K, D] */
  const void* v1;           /* DEVICE [B, H, N, K, D] */
  const void* k2;           /* DEVICE [B, H, M, K, D] */
  const void* v2;           /* DEVICE [B, H, M, K, D] */
  void* out;                /* DEVICE, written [B, H, N, M, D] */
  float* lse;               /* DEVICE, written [B, H, N, M] */
  int32_t reuse_lists;      /* unused (no lists); keep 0 */
  int32_t n_events;         /* number of stages to time (0 = off) */
  void* const* events;      /* HOST array of 2*n_events hipEvent_t (see above) */
} floyd_fwd_args;

typedef struct {
  int32_t dtype;
  int32_t B, H, N, M, K, D;
  float scale;
  const void* q;            /* DEVICE, as in the forward */
  const void* k1;
  const void* v1;
  const void* k2;
  const void* v2;
  const void* out;          /* DEVICE, the forward output */
  const void* dout;         /* DEVICE, its gradient [B, H, N, M, D] */
  const float* lse;         /* DEVICE, the forward LSE */
  void* dq;                 /* DEVICE, written, like q */
  void* dk1;                /* DEVICE, written, like k1 */
  void* dv1;                /* DEVICE, written, like v1 */
  void* dk2;                /* DEVICE, written, like k2 */
  void* dv2;                /* DEVICE, written, like v2 */
  int32_t reuse_lists;      /* unused; keep 0 */
  int32_t n_events;
  void* const* events;
} floyd_bwd_args;

TSA_API int floyd_fwd_workspace_size(const floyd_fwd_args* args, size_t* bytes);
TSA_API int floyd_fwd(const floyd_fwd_args* args, void* workspace, size_t workspace_bytes,
                      void* stream);
TSA_API int floyd_bwd_workspace_size(const floyd_bwd_args* args, size_t* bytes);
TSA_API int floyd_bwd(const floyd_bwd_args* args, void* workspace, size_t workspace_bytes,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOP_SELECTED_ATTENTION_H */
