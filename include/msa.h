/*
 * msa.h -- C ABI of the MSA (MiniMax Sparse Attention) hot path on AMD MI355X (gfx950).
 *
 * MSA is two-branch block-sparse attention layered on GQA (MSA guide,
 * ai-tool-zukan.com/minimax-msa-guide, section "MiniMax MSAとは何か").  The three
 * compute entry points follow the decomposition the same page gives in its
 * pseudocode figure (section "Index BranchとMain Branchの役割分担"):
 *
 *   msa_index_select()            score -> top_k(k) -> ensure_local_block
 *   msa_build_block_query_lists() regroup the selection KV-block-outer
 *                                 (tnkblog.net MiniMax M3 MSA post, section "MSA の実装")
 *   msa_attend()                  exact softmax attention over the selected blocks
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are dense, row-major, and live in device memory unless stated.
 *   Every tensor pointer must be 16-byte aligned.
 * - Sequences are packed ("varlen"): sequence b owns query rows
 *   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 *   cu_seqlens_k[b+1]-1.  Its Lq_b queries are the LAST Lq_b of its Lk_b
 *   positions: query i sits at position Lk_b - Lq_b + i (prefill: Lq = Lk;
 *   decode: Lq = 1 at position Lk - 1).  Requires 0 <= Lq_b <= Lk_b.
 *   cu_seqlens_* are int32 device arrays of batch + 1 entries.
 * - KV block beta of a sequence is its positions [128*beta, 128*beta + 127];
 *   blocks start at position 0 of every sequence.
 * - Query head h belongs to GQA group h / (num_q_heads / num_kv_heads); there
 *   is one index-query head per group and one shared index-key head.
 * - Ownership: the caller allocates every buffer, workspace included; the
 *   library never allocates, frees or keeps device memory.  All work is
 *   enqueued on `stream` (a hipStream_t; NULL = the default stream) with no
 *   host synchronisation; buffers must stay alive until the stream has passed
 *   the call.  Outputs are bitwise deterministic for identical inputs.
 * - No queries (total_q == 0): msa_index_select and msa_attend enqueue
 *   nothing; msa_build_block_query_lists still writes all-zero offsets.
 * - Errors: every argument is validated on the host before anything is
 *   launched; a call that returns an error has enqueued nothing.  A failed
 *   HIP launch returns MSA_ERR_HIP (msa_last_error() gives HIP's message).
 *   Device data that breaks the stated layout gives undefined results.  For
 *   the two kinds of device data a caller typically writes by hand -- block
 *   ids in `sel` (out of range, repeated, or after the query's block) and
 *   block_table entries -- the kernels bound every address they derive from
 *   them, so such data cannot make a kernel read or write outside its
 *   buffers.  cu_seqlens_q / cu_seqlens_k are trusted: they must be
 *   non-decreasing, start at 0, end at total_q / total_k, and agree with
 *   max_q_len / max_k_len and 0 <= Lq_b <= Lk_b; other values are undefined
 *   behaviour (kernels may then access memory outside the buffers).
 * - Debugging: with the environment variable MSA_DEBUG_SYNC set (to anything
 *   but "" or "0"; read at every call), each call first copies its
 *   cu_seqlens to the host and rejects values that break the rules above
 *   (MSA_ERR_BAD_DIMS, nothing enqueued), and every kernel stage is followed
 *   by a wait on the stream and an error check whose message names the
 *   stage (MSA_ERR_HIP).  It blocks the host; not for use under graph capture.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 3
#define MSA_BLOCK_SIZE 128  /* B_k, MSA guide table in section "ブロック単位選択の数値設計" */
#define MSA_MAX_TOP_K 32

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  MSA_ERR_BAD_DIMS = 2,            /* inconsistent or out-of-range sizes */
  MSA_ERR_UNSUPPORTED = 3,         /* valid MSA, but not a size this build implements */
  MSA_ERR_ALIGNMENT = 4,           /* a tensor pointer is not 16-byte aligned */
  MSA_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below msa_workspace_size() */
  MSA_ERR_HIP = 6                  /* a HIP runtime call or launch failed */
} msa_status_t;

typedef enum msa_op {
  MSA_OP_INDEX_SELECT = 0,
  MSA_OP_BUILD_LISTS = 1,
  MSA_OP_ATTEND = 2,
  MSA_OP_INDEX_PROJECT = 3
} msa_op_t;

/* Problem sizes; passed by pointer to every call.  All fields are host values. */
typedef struct msa_dims {
  int32_t batch;          /* number of packed sequences, 1 .. 65535 */
  int32_t num_q_heads;    /* Hq; Hq / Hkv must be a power of two <= 32 */
  int32_t num_kv_heads;   /* Hkv = G = number of GQA groups = number of index-query heads */
  int32_t head_dim;       /* d in {64, 128} */
  int32_t index_dim;      /* d_idx in {32, 64, 128} */
  int32_t block_size;     /* must be 128 */
  int32_t top_k;          /* blocks per (query, group) INCLUDING the forced local block, 1..32 */
  float softmax_scale;    /* 0 -> 1/sqrt(head_dim); else finite and > 0 */
  int64_t total_q;        /* sum of Lq_b; < 2^26 (list entries pack row * 32 + slot) */
  int64_t total_k;        /* sum of Lk_b */
  int32_t max_q_len;      /* max_b Lq_b (host-known upper bound; sizes launch grids) */
  int32_t max_k_len;      /* max_b Lk_b (host-known upper bound; sizes launch grids) */
  int32_t q_chunk;        /* query rows processed per internal pass; 0 -> library default.
                             Bounds the workspace; results do not depend on it. */
  int32_t kv_pages;       /* 0: contiguous key rows (sequence b owns rows cu_seqlens_k[b] ..);
                             > 0: paged key cache of this many 128-row pages (see below) */
  const int32_t* block_table;   /* paged only: device int32 [batch, max_blocks_per_seq]; block
                                   beta of sequence b is page block_table[b][beta] */
  int32_t max_blocks_per_seq;   /* paged only: row stride of block_table, >= ceil(max_k_len/128) */
  int32_t flags;          /* 0, or MSA_FLAG_COMPACT_PARTIALS; other bits must be 0 */
} msa_dims_t;

/*
 * MSA_FLAG_COMPACT_PARTIALS: the Main Branch's per-(query, head, block)
 * softmax partials, which it writes and merges inside msa_attend (and
 * msa_attend_fp8 / _q8kv4 / _noalloc), are kept as 2 * head_dim + 8 bytes
 * instead of 4 * head_dim + 8: the block's log-sum-exp w = m + log2 l and a
 * power-of-two exponent E in fp32, and O / l * 2^-E in fp16 (magnitudes below
 * 1, 11 significant bits; E is chosen per row from its largest |O|).  This
 * roughly halves the Main Branch's memory traffic on prefill-shaped steps.
 * Each stored value is off by at most 2^-11 of its row's largest |O / l|
 * (fp16 rounding), so the merged output moves by at most 2^-11 of the
 * largest |v| the query attends to, on the order of the bf16 rounding of the
 * output itself.  It applies where msa_attend_reads_lists()
 * is 1 (decode-shaped steps keep fp32 partials, a small part of their
 * bytes), lowers msa_workspace_size(MSA_OP_ATTEND) accordingly, and is not
 * supported by msa_attend_with_mass (MSA_ERR_UNSUPPORTED), whose block
 * masses read the fp32 (m, l).  Without the flag the partials are fp32.
 */
#define MSA_FLAG_COMPACT_PARTIALS 1

/*
 * Paged key cache (kv_pages > 0).  A page holds one 128-token KV block, the
 * unit the selection works in, so block beta of sequence b lives in page
 * block_table[b][beta]: key position j of sequence b is row
 * 128 * block_table[b][j / 128] + j % 128 of k, v and k_idx (and of k_idx8;
 * the fp8 key exponents k_exp are then one per page, [kv_pages]).  total_k
 * must equal 128 * kv_pages (the caches' row count); cu_seqlens_k still gives
 * each sequence's length (its differences), its offsets are not used.  Every
 * call that reads or writes key rows follows the table; block_table entries
 * of a sequence's blocks must be distinct valid pages.  The table is read on
 * the device, so it is not validated: an entry outside [0, kv_pages) is
 * clamped into that range (the results are then wrong, but no access leaves
 * the caches).  The table must stay allocated until the call's work ends.
 */

/* Bytes of workspace the call `op` needs for `dims` (same dims as the call).
 * Returns MSA_ERR_* on invalid dims, else MSA_OK and *bytes. */
msa_status_t msa_workspace_size(const msa_dims_t* dims, msa_op_t op, size_t* bytes);

/*
 * Index Branch: per (query, group), the selected KV blocks.
 *
 * Computes, for every query row r at position p of its sequence and every
 * group g (MSA guide, section "2段階構造の中身"; roles of the two index
 * projections in section "Index BranchとMain Branchの役割分担"):
 *   s[j]      = q_idx[r, g, :] . k_idx[j, :] for the visible keys j <= p,
 *               accumulated in fp32 from bf16 inputs;
 *   S[beta]   = max of s over the tokens of block beta (max-pooling);
 *   sel[r, g] = { beta(p) } plus the top_k - 1 earlier blocks beta < beta(p)
 *               with the largest S (ties: lower beta first); when fewer than
 *               top_k - 1 earlier blocks exist, all of them.  The query's own
 *               block is always in (section "クエリを含むローカルブロックの強制取り込み")
 *               and counts toward top_k, so top_k = 16 keeps the fixed budget of
 *               16 * 128 = 2,048 tokens (table in section "ブロック単位選択の数値設計").
 *   The selection is shared by all query heads of the group and made
 *   independently per group (section "GQAグループ単位の選択共有とは").
 *
 * q_idx     bf16  [total_q, num_kv_heads, index_dim]
 * k_idx     bf16  [total_k, index_dim]
 * sel       int32 [total_q, num_kv_heads, top_k]  out: ascending block ids, -1 padded
 * sel_score fp32  [total_q, num_kv_heads, top_k]  out, optional (NULL): S of each
 *           selected block, +inf for the local block, NaN for padding
 * workspace >= msa_workspace_size(dims, MSA_OP_INDEX_SELECT) bytes
 * When max_q_len * num_kv_heads > 128 (the prefill kernel, which scores all
 * groups of a query in one workgroup) num_kv_heads must be <= 512, else
 * MSA_ERR_UNSUPPORTED.
 */
msa_status_t msa_index_select(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t* sel, float* sel_score, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * KV-block-outer regrouping: for every (sequence b, group g, block beta) the
 * queries whose selection holds beta (tnkblog.net MiniMax M3 MSA post,
 * section "MSA の実装": KV block as the outer loop, gathering the queries that
 * hit it; the same order in the wiki repost of the CSDN article, section
 * "MiniMax Sparse Attention（MSA）", item 3).
 *
 * Bucket u = (b * num_kv_heads + g) * nb_max + beta, nb_max = ceil(max_k_len / 128).
 * block_offsets int32 [batch * num_kv_heads * nb_max + 1]  out: CSR offsets
 * block_entries int32 [total_q * num_kv_heads * top_k]     out: for bucket u,
 *               entries block_offsets[u] .. block_offsets[u+1]-1 hold
 *               row * 32 + slot with sel[row, g, slot] == beta, rows ascending.
 *               Entries past block_offsets[U] are left untouched.
 * sel           as produced by msa_index_select (any valid selection works).
 * workspace >= msa_workspace_size(dims, MSA_OP_BUILD_LISTS) bytes
 */
msa_status_t msa_build_block_query_lists(const msa_dims_t* dims, const int32_t* sel,
                                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                         int32_t* block_offsets, int32_t* block_entries,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Main Branch: exact softmax attention of every query head over the visible
 * keys of its group's selected blocks (MSA guide, sections "MiniMax MSAとは何か"
 * and "2段階構造の中身"): out[r, h] = sum_j softmax_j(scale * q[r,h] . k[j,g]) v[j,g]
 * over J = { j <= p : beta(j) in sel[r, g] }.  Run KV-block-outer: each block's
 * K/V is staged on chip once per pass and serves every gathered query; the
 * per-(query, head, block) softmax partials are merged by log-sum-exp.
 *
 * Decode-shaped steps (max_q_len <= 8 new tokens per sequence): a selected
 * block is hit by at most a few queries, so the call works per (query, slot)
 * straight from sel and does not read the lists; msa_attend_reads_lists()
 * tells which case dims fall in, and where it returns 0 the lists may be NULL
 * and msa_build_block_query_lists need not run.
 *
 * q        bf16 [total_q, num_q_heads, head_dim]
 * k, v     bf16 [total_k, num_kv_heads, head_dim]
 * sel, block_offsets, block_entries: as from the two calls above (same dims)
 * out      bf16 [total_q, num_q_heads, head_dim]  out
 * lse      fp32 [total_q, num_q_heads]  out, optional (NULL): natural-log
 *          log-sum-exp of the scaled logits over J
 * workspace >= msa_workspace_size(dims, MSA_OP_ATTEND) bytes
 */
msa_status_t msa_attend(const msa_dims_t* dims, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* sel, const int32_t* block_offsets,
                        const int32_t* block_entries, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Index projections: the two projection matrices the Index Branch adds to a
 * GQA layer (MSA guide, section "Index BranchとMain Branchの役割分担": one
 * index-query head per group, one shared index-key head), applied to the
 * layer input of the new tokens:
 *   q_idx[r, g, :] = x[r, :] . W_q[g * index_dim + c, :]  (c = 0 .. index_dim-1)
 *   k_idx[row(r), :] = x[r, :] . W_k[c, :]
 * accumulated in fp32 and rounded to bf16 (nearest even).  x has one row per
 * query row r; row(r) is the key row of that token in its sequence
 * (cu_seqlens_k[b] + Lk_b - Lq_b + i for the i-th query of sequence b), so a
 * prefill (Lq = Lk) writes every key row and a decode step writes each
 * sequence's new keys after its cached ones; other key rows are untouched.
 * No bias.  The pages give no layer width: model_dim is a parameter.
 *
 * model_dim D: multiple of 64, 64 .. 65536 (else MSA_ERR_UNSUPPORTED)
 * x      bf16 [total_q, D]
 * w_q    bf16 [num_kv_heads * index_dim, D]   (out_features x in_features)
 * w_k    bf16 [index_dim, D]
 * q_idx  bf16 [total_q, num_kv_heads, index_dim]  out
 * k_idx  bf16 [total_k, index_dim]                out (the new tokens' rows)
 * workspace  16-byte aligned; msa_workspace_size(dims, MSA_OP_INDEX_PROJECT)
 *   bytes is what the fastest launch uses: fp32 tiles of slices of the sum
 *   over model_dim, taken by different workgroups.  Steps of up to 512
 *   tokens always split the sum and must be given at least that much (a
 *   few MiB; else MSA_ERR_NULL_ARG or MSA_ERR_WORKSPACE_TOO_SMALL).  Larger
 *   steps split it only while the GPU would otherwise be underfilled (up to
 *   a few thousand tokens; at most 64 MiB) and only if the workspace holds
 *   the slices; NULL or a smaller workspace runs them unsplit.  Partial sums
 *   are added in a fixed order: results are deterministic for a given
 *   workspace size (a split and an unsplit run differ by fp32 rounding).
 * total_q == 0 enqueues nothing.
 */
msa_status_t msa_index_project(const msa_dims_t* dims, int32_t model_dim, const void* x,
                               const void* w_q, const void* w_k, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, void* q_idx, void* k_idx,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Quantised Index Branch (optional; the bf16 calls above are the reference
 * path).  The pages note that the production model runs the sparse
 * attention's indexer with 8-bit queries and 8-bit keys (dot-ai.myuuu.co.jp
 * article on MiniMax M3.1 Flash, section "MiniMax M3.1 Flashとは？428Bの
 * MoEモデルがウェイト公開", on the model card's quantisation notes: indexer
 * and Main Branch "Q8KV8", moving to 4-bit keys).  Format and scaling are this library's reading:
 *   - codes are OCP FP8 E4M3 (bias 7, largest finite 448, no infinities);
 *   - scales are powers of two stored as E8M0 bytes (value = 2^(byte - 127));
 *   - one scale per (query row, group) of q_idx, one per (sequence, 128-token
 *     KV block) of k_idx;
 *   - a row's or block's exponent e is the smallest integer with
 *     max|x| * 2^-e <= 448, clamped to [-127, 127] (0 for an all-zero row or
 *     block); code = round-to-nearest-even E4M3 of x * 2^-e.
 * Non-finite index inputs give unspecified codes.
 *
 * msa_index_quantize_fp8: bf16 index projections -> codes + exponents.
 *   Either side may be left out by passing NULL as its input (its outputs
 *   are then not touched): a decode step quantises its new index queries
 *   against an index-key cache quantised once when it was written.
 *   q_idx   bf16 [total_q, num_kv_heads, index_dim]   or NULL
 *   k_idx   bf16 [total_k, index_dim]                 or NULL
 *   q_idx8  uint8 E4M3 [total_q, num_kv_heads, index_dim]  out
 *   q_exp   uint8 E8M0 [total_q, num_kv_heads]              out (no alignment needed)
 *   k_idx8  uint8 E4M3 [total_k, index_dim]                 out
 *   k_exp   uint8 E8M0 [batch, nb_max], nb_max = ceil(max_k_len / 128)   out;
 *           k_exp[b, beta] scales keys cu_k[b] + 128 beta .. of sequence b;
 *           blocks past a sequence's end get 127.  Paged cache: [kv_pages],
 *           one per page; only the pages of the sequences' blocks are written.
 *   No workspace.  With total_q == 0 only the keys are quantised.  Keys are
 *   quantised per whole block, so a key cache quantised this way is
 *   re-quantised block by block as blocks fill (the selection never scores a
 *   query's own, still filling, block).
 *
 * msa_index_select_fp8: msa_index_select on the dequantised values
 *   q = decode(q_idx8) * 2^(q_exp - 127), k = decode(k_idx8) * 2^(k_exp - 127).
 *   Token dot products of the codes run on the fp8 matrix cores, which sum
 *   each group of 8 products in fixed point aligned to the group's largest
 *   product (13 bits below its leading bit) and add the groups in fp32: a
 *   token score is within 2^-10 * sum_c |q_c k_c| of the exact dot product of
 *   the dequantised values.  Since a block's scale is common to its keys, the
 *   block score is 2^(eq + ek) * max_j (q8 . k8_j), applied exactly.  Selection rule, tie
 *   rule, outputs and workspace (msa_workspace_size with MSA_OP_INDEX_SELECT)
 *   are those of msa_index_select; sel_score holds the dequantised block
 *   scores.  Requires ceil(max_k_len / 128) <= 16384, and num_kv_heads <= 256
 *   when max_q_len * num_kv_heads > 128 (else MSA_ERR_UNSUPPORTED).
 */
msa_status_t msa_index_quantize_fp8(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                                    const int32_t* cu_seqlens_k, void* q_idx8, uint8_t* q_exp,
                                    void* k_idx8, uint8_t* k_exp, void* stream);
msa_status_t msa_index_select_fp8(const msa_dims_t* dims, const void* q_idx8, const uint8_t* q_exp,
                                  const void* k_idx8, const uint8_t* k_exp,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t* sel, float* sel_score, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Index Branch with 4-bit index keys ("Q8KV4").  The pages state that the
 * production indexer moves from 8-bit keys to 4-bit keys, queries staying at
 * 8 bits (dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
 * "MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開", on the model card's
 * quantisation notes).  Format and scaling are this library's reading:
 *   - queries exactly as msa_index_quantize_fp8 (E4M3, one E8M0 exponent per
 *     (query row, group));
 *   - key codes are OCP FP4 E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *     negatives), two per byte, element 2i in the low nibble;
 *   - one E8M0 exponent per 32 consecutive elements of a key row (the OCP
 *     microscaling block): e is the smallest integer with
 *     max|x| * 2^-e <= 6, clamped to [-127, 127] (0 for an all-zero group);
 *     code = nearest E2M1 value of x * 2^-e, ties to the even code, with the
 *     sign bit of x.
 * Non-finite index inputs give unspecified codes.
 *
 * msa_index_quantize_q8k4: bf16 index projections -> codes + exponents.
 *   Either side may be left out by passing NULL as its input (its outputs
 *   are then not touched).
 *   q_idx   bf16 [total_q, num_kv_heads, index_dim]   or NULL
 *   k_idx   bf16 [total_k, index_dim]                 or NULL
 *   q_idx8  uint8 E4M3 [total_q, num_kv_heads, index_dim]  out
 *   q_exp   uint8 E8M0 [total_q, num_kv_heads]              out (no alignment needed)
 *   k_idx4  uint8 [total_k, index_dim / 2] packed E2M1    out
 *   k_exp4  uint8 E8M0 [total_k, index_dim / 32]          out
 *           Rows as in k_idx (contiguous, or 128 * page + j when paged).
 *           Only the rows of the sequences' keys are written: keys are
 *           quantised row by row, so a cache can be extended a token at a time.
 *   No workspace.  q_idx, k_idx, q_idx8, k_idx4 and k_exp4 16-byte aligned.
 *
 * msa_index_select_q8k4: msa_index_select on the dequantised values
 *   q = decode(q_idx8) * 2^(q_exp - 127),
 *   k[j, c] = decode4(k_idx4[j, c]) * 2^(k_exp4[j, c / 32] - 127).
 *   The key exponents scale the products inside gfx950's microscaled matrix
 *   instructions (E2M1 x E4M3), summed as for msa_index_select_fp8, so a
 *   token score is within 2^-10 * sum_c |q_c k_c| of the exact value; the
 *   query exponent is applied to the block maximum.  Selection rule, tie
 *   rule, outputs and workspace are those of msa_index_select; sel_score
 *   holds the dequantised block scores.  num_kv_heads <= 256 when
 *   max_q_len * num_kv_heads > 128 (else MSA_ERR_UNSUPPORTED).
 */
msa_status_t msa_index_quantize_q8k4(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                                     const int32_t* cu_seqlens_k, void* q_idx8, uint8_t* q_exp,
                                     void* k_idx4, uint8_t* k_exp4, void* stream);
msa_status_t msa_index_select_q8k4(const msa_dims_t* dims, const void* q_idx8, const uint8_t* q_exp,
                                   const void* k_idx4, const uint8_t* k_exp4,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t* sel, float* sel_score, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * KL-alignment target of the Index Branch, forward only.  The pages train the
 * non-differentiable top-k by pulling the distribution of the Index Branch's
 * block scores towards the distribution of blocks the Main Branch's exact
 * attention relied on, through a KL divergence (MSA guide, sections
 * "非微分的な選択をどう学習させるか（KLダイバージェンス）" and "選択を学習可能にするKL損失").
 * This library's reading, per (query, group), over the selected blocks:
 *   P(s) = Main-Branch attention mass on selected slot s, averaged over the
 *          group's query heads (sums to 1 over the selection);
 *   Q(s) = softmax of the selected blocks' index scores, the local block
 *          scored on its visible tokens (no temperature);
 *   KL   = sum_s P(s) (log P(s) - log Q(s)).
 *
 * msa_attend_with_mass: msa_attend plus
 *   block_mass fp32 [total_q, num_kv_heads, top_k]  out: P, aligned with sel; 0 for padding.
 * msa_index_kl: from the Index Branch inputs, the selection and its scores
 *   (msa_index_select with sel_score, bf16 path) and block_mass:
 *   log_q fp32 [total_q, num_kv_heads, top_k]  out, optional (NULL): log Q, NaN for padding
 *   kl    fp32 [total_q, num_kv_heads]         out
 *   No workspace.  total_q == 0 enqueues nothing.
 */
msa_status_t msa_attend_with_mass(const msa_dims_t* dims, const void* q, const void* k,
                                  const void* v, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, const int32_t* sel,
                                  const int32_t* block_offsets, const int32_t* block_entries,
                                  void* out, float* lse, float* block_mass, void* workspace,
                                  size_t workspace_bytes, void* stream);
msa_status_t msa_index_kl(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* sel, const float* sel_score, const float* block_mass,
                          float* log_q, float* kl, void* stream);

/*
 * Quantised Main Branch (optional; msa_attend is the reference path).  The
 * pages note that the production model runs the Main Branch, like the
 * indexer, with 8-bit queries and 8-bit keys/values (dot-ai.myuuu.co.jp
 * article on MiniMax M3.1 Flash, section "MiniMax M3.1 Flashとは？428Bの
 * MoEモデルがウェイト公開", on the model card's quantisation notes: "Q8KV8").
 * Format and scale rule as for msa_index_quantize_fp8 (OCP E4M3 codes,
 * E8M0 power-of-two scales, smallest exponent e with max|x| * 2^-e <= 448,
 * round to nearest even); granularity (this library's reading): one scale
 * per (query row, head) of q, one per (sequence block, KV head) of k and v.
 *
 * msa_main_quantize_fp8: bf16 q / k / v -> codes + exponents.  Any of q, k, v
 *   may be NULL (its outputs are then not touched): a decode step quantises
 *   its new queries against a key/value cache quantised when written.
 *   q     bf16 [total_q, num_q_heads, head_dim]   or NULL
 *   k, v  bf16 [total_k, num_kv_heads, head_dim]  or NULL
 *   q8    uint8 E4M3 [total_q, num_q_heads, head_dim]  out
 *   q_exp uint8 E8M0 [total_q, num_q_heads]             out (no alignment needed)
 *   k8, v8 uint8 E4M3 [total_k, num_kv_heads, head_dim]  out
 *   k_exp, v_exp uint8 E8M0 [batch, nb_max, num_kv_heads] out, nb_max =
 *          ceil(max_k_len / 128); blocks past a sequence's end get 127.
 *          Paged cache: [kv_pages, num_kv_heads], one per (page, head), and
 *          only the pages of the sequences' blocks are written.
 * msa_attend_fp8: msa_attend on the dequantised values (the same exact
 *   softmax over the selected blocks; the codes are dequantised exactly into
 *   bf16 operands while loading, so the arithmetic is msa_attend's).  Same
 *   selection, lists, outputs, workspace and routing as msa_attend.
 */
msa_status_t msa_main_quantize_fp8(const msa_dims_t* dims, const void* q, const void* k,
                                   const void* v, const int32_t* cu_seqlens_k, void* q8,
                                   uint8_t* q_exp, void* k8, uint8_t* k_exp, void* v8,
                                   uint8_t* v_exp, void* stream);
msa_status_t msa_attend_fp8(const msa_dims_t* dims, const void* q8, const uint8_t* q_exp,
                            const void* k8, const uint8_t* k_exp, const void* v8,
                            const uint8_t* v_exp, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const int32_t* sel,
                            const int32_t* block_offsets, const int32_t* block_entries, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_attend without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It computes exactly what msa_attend computes, with
 * the same kernels, and allocates nothing: the per-(query, head, block)
 * partials live in a scratch array the library holds in device memory, one
 * copy of MSA_NOALLOC_SCRATCH_BYTES per GPU for the life of the process,
 * located on its first call on a device (the device of `stream`).
 * - Sizes: the call needs msa_workspace_size(dims, MSA_OP_ATTEND) <=
 *   MSA_NOALLOC_SCRATCH_BYTES, else it returns MSA_ERR_WORKSPACE_TOO_SMALL
 *   and enqueues nothing; dims->q_chunk lowers that size (results do not
 *   depend on it).  A decode step of 32 sequences with 64 query heads and
 *   top_k 16 needs about 17 MiB.
 * - Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents; nothing in it needs to start at zero (every partial
 *   the call reads, it has written).  Calls that overlap on one GPU (on
 *   different streams, or from different host threads without ordering)
 *   race on the scratch and give undefined results.
 * Other arguments, errors and stream semantics as msa_attend.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
msa_status_t msa_attend_noalloc(const msa_dims_t* dims, const void* q, const void* k,
                                const void* v, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* sel,
                                const int32_t* block_offsets, const int32_t* block_entries,
                                void* out, float* lse, void* stream);

/* Query rows that msa_attend and its variants process per internal pass for
 * these dims (dims->q_chunk when set, else the library's choice, which keeps
 * the workspace under 72 GiB): a call makes ceil(total_q / rows) passes, and
 * a KV block whose query list spans several passes is staged once per pass.
 * A negative msa_status_t for invalid dims. */
int64_t msa_attend_pass_rows(const msa_dims_t* dims);

/* 1 if msa_attend / msa_attend_with_mass / msa_attend_fp8 read block_offsets and
 * block_entries for these dims, 0 if they work from sel alone (decode-shaped
 * steps), a negative msa_status_t for invalid dims. */
int32_t msa_attend_reads_lists(const msa_dims_t* dims);

/*
 * Main Branch with 4-bit keys and values ("Q8KV4").  The pages state that
 * the production indexer and Main Branch move from 8-bit queries and
 * keys/values to 8-bit queries and 4-bit keys/values (dot-ai.myuuu.co.jp
 * article on MiniMax M3.1 Flash, section "MiniMax M3.1 Flashとは？428Bの
 * MoEモデルがウェイト公開", on the model card's quantisation notes).  This
 * library's reading: queries as msa_main_quantize_fp8 (E4M3, one E8M0
 * exponent per (query row, head)); keys and values in the 4-bit index keys'
 * format (see msa_index_quantize_q8k4): OCP E2M1 codes, two per byte
 * (element 2i in the low nibble), one E8M0 exponent per 32 consecutive
 * elements of every (key, KV head) row, e = smallest integer with
 * max|x| * 2^-e <= 6 clamped to [-127, 127], nearest E2M1 value of x * 2^-e
 * with ties to the even code.
 *
 * msa_main_quantize_q8kv4: bf16 q / k / v -> codes + exponents; any of q, k,
 *   v may be NULL (its outputs are then not touched): a decode step
 *   quantises its new queries against a cache quantised when written.
 *   q8      uint8 E4M3 [total_q, num_q_heads, head_dim]        out
 *   q_exp   uint8 E8M0 [total_q, num_q_heads]                   out
 *   k4, v4  uint8 [total_k, num_kv_heads, head_dim / 2]         out
 *   k_exp4, v_exp4  uint8 E8M0 [total_k, num_kv_heads, head_dim / 32]  out
 *   Rows as in k (page rows when paged); only the sequences' keys are
 *   written.  q, k, v, q8, k4, v4, k_exp4, v_exp4 16-byte aligned.
 * msa_attend_q8kv4: msa_attend on the dequantised q, k, v.  The kernels
 *   dequantise exactly into bf16 operands (an E2M1 value times a power of
 *   two is a bf16 value) and then compute what msa_attend computes; lists,
 *   outputs, workspace and errors as msa_attend.  q8, k4, v4, k_exp4 and
 *   v_exp4 16-byte aligned (MSA_ERR_ALIGNMENT otherwise).
 */
msa_status_t msa_main_quantize_q8kv4(const msa_dims_t* dims, const void* q, const void* k,
                                     const void* v, const int32_t* cu_seqlens_k, void* q8,
                                     uint8_t* q_exp, void* k4, uint8_t* k_exp4, void* v4,
                                     uint8_t* v_exp4, void* stream);
msa_status_t msa_attend_q8kv4(const msa_dims_t* dims, const void* q8, const uint8_t* q_exp,
                              const void* k4, const uint8_t* k_exp4, const void* v4,
                              const uint8_t* v_exp4, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, const int32_t* sel,
                              const int32_t* block_offsets, const int32_t* block_entries, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* msa_status_string(msa_status_t status);

/* Message of the last MSA_ERR_HIP (or validation detail) on the calling thread. */
const char* msa_last_error(void);

/* MSA_ABI_VERSION of the loaded library. */
int32_t msa_abi_version(void);

/*
 * Per-kernel timing, a measuring aid (not part of the pages' method).  While
 * enabled, every kernel stage a call launches is bracketed by two hipEvents
 * recorded on the call's stream.  Stage ids: 0 index_select_prefill (scores + top-k),
 * 1 index_score_decode, 2 topk_select, 3 build_lists (all list kernels),
 * 4 attend_blocks, 5 merge_partials, 6 quantize_index_fp8,
 * 7 index_select_prefill_fp8, 8 index_score_decode_fp8, 9 index_project, 10 block_mass,
 * 11 index_kl, 12 quantize_main_fp8, 13 quantize_index_q8k4,
 * 14 index_select_prefill_q8k4, 15 index_score_decode_q8k4, 16 quantize_main_q8kv4.
 * msa_profile_collect() waits for every
 * recorded event (it blocks the host), writes the summed milliseconds and the
 * launch count per stage into caller arrays of MSA_PROFILE_KERNELS entries,
 * and forgets the records.  Events are host-side HIP objects kept in a pool
 * for the life of the process; no device memory is allocated.
 */
/*
 * A second measuring aid: a plain streaming kernel that reads read_bytes from
 * src and writes ratio * read_bytes to dst (ratio 0..4; 0 reads only), each
 * byte once, with every instruction covering 1 KiB of consecutive bytes.  Its
 * rate is the ceiling a kernel with the same read:write mix can reach on the
 * GPU at hand (the Main Branch's attend pass writes about two bytes per byte
 * read; its merge pass reads almost only).  read_bytes: a positive multiple
 * of 16; dst: ratio * read_bytes bytes (NULL allowed for ratio 0); sink: at
 * least 4 * MSA_HBM_STREAM_MAX_WORKGROUPS bytes (practically never written).
 * All pointers device memory, 16-byte aligned.  Enqueued on `stream`.
 */
#define MSA_HBM_STREAM_MAX_WORKGROUPS 2048
msa_status_t msa_hbm_stream(const void* src, size_t read_bytes, int32_t ratio, void* dst,
                            void* sink, void* stream);

#define MSA_PROFILE_KERNELS 17
msa_status_t msa_profile_enable(int32_t enable);
msa_status_t msa_profile_collect(float* total_ms, int32_t* launches);
const char* msa_profile_kernel_name(int32_t id);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
