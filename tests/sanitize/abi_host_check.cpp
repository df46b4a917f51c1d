// Host-side checks of the MSA C ABI, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_abi_host_sanitized.py;
// no GPU needed).  Every call here is rejected by host validation before any
// HIP call, or is a pure size query, so the sanitizers watch the library's
// own argument checks and size arithmetic: dims near every limit, NULL and
// misaligned pointers, undersized workspaces, unknown flags.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "msa.h"

static int failures = 0;

#define EXPECT(cond, what)                                                  \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, what,     \
              msa_last_error());                                            \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static msa_dims_t base_dims(void) {
  msa_dims_t d;
  memset(&d, 0, sizeof d);
  d.batch = 1;
  d.num_q_heads = 64;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.index_dim = 128;
  d.block_size = 128;
  d.top_k = 16;
  d.total_q = 32768;
  d.total_k = 32768;
  d.max_q_len = 32768;
  d.max_k_len = 32768;
  return d;
}

int main(void) {
  EXPECT(msa_abi_version() == MSA_ABI_VERSION, "abi version");
  EXPECT(sizeof(msa_dims_t) == 80, "struct size");
  for (int s = 0; s <= 6; ++s) {
    msa_status_t st;
    memcpy(&st, &s, sizeof st);
    EXPECT(strncmp(msa_status_string(st), "MSA_", 4) == 0, "status string");
  }
  // a C caller may pass any int where the ABI takes an enum
  {
    int bad[] = {-1, 7, 99, 1 << 30};
    for (int i = 0; i < 4; ++i) {
      msa_status_t s;
      memcpy(&s, &bad[i], sizeof s);
      EXPECT(strcmp(msa_status_string(s), "MSA_ERR_UNKNOWN") == 0, "unknown status");
      msa_op_t op;
      memcpy(&op, &bad[i], sizeof op);
      msa_dims_t d = base_dims();
      size_t bytes = 0;
      EXPECT(msa_workspace_size(&d, op, &bytes) == MSA_ERR_BAD_DIMS, "unknown op");
    }
  }

  // size queries over a sweep of shapes, including the limits
  const int64_t lens[] = {0, 1, 127, 128, 129, 4096, 131072, 1 << 20, 2080768};
  const int32_t topks[] = {1, 2, 16, 31, 32};
  const int32_t chunks[] = {0, 1, 100, 65536};
  for (size_t i = 0; i < sizeof lens / sizeof lens[0]; ++i)
    for (size_t j = 0; j < sizeof topks / sizeof topks[0]; ++j)
      for (size_t c = 0; c < sizeof chunks / sizeof chunks[0]; ++c)
        for (int flags = 0; flags <= 1; ++flags) {
          msa_dims_t d = base_dims();
          d.total_q = d.total_k = lens[i] < 1 ? 1 : lens[i];
          d.max_q_len = d.max_k_len = (int32_t)d.total_q;
          d.top_k = topks[j];
          d.q_chunk = chunks[c];
          d.flags = flags;
          for (int op = 0; op <= 3; ++op) {
            size_t bytes = 0;
            msa_status_t st = msa_workspace_size(&d, (msa_op_t)op, &bytes);
            EXPECT(st == MSA_OK || st == MSA_ERR_UNSUPPORTED, "workspace size");
            if (st == MSA_OK && op != MSA_OP_INDEX_PROJECT) EXPECT(bytes > 0, "nonzero workspace");
          }
          const int64_t rows = msa_attend_pass_rows(&d);
          EXPECT(rows < 0 || (rows >= 1 && rows <= d.total_q), "pass rows");
          EXPECT(msa_attend_reads_lists(&d) >= -6, "reads lists");
        }

  // decode batches up to the grid limit
  {
    msa_dims_t d = base_dims();
    d.batch = 65535;
    d.total_q = 65535;
    d.total_k = (int64_t)65535 * 128;
    d.max_q_len = 1;
    d.max_k_len = 128;
    size_t bytes = 0;
    EXPECT(msa_workspace_size(&d, MSA_OP_INDEX_SELECT, &bytes) == MSA_OK, "decode batch 65535");
    d.batch = 65536;
    EXPECT(msa_workspace_size(&d, MSA_OP_INDEX_SELECT, &bytes) == MSA_ERR_UNSUPPORTED, "batch 65536");
  }

  // invalid dims of every kind
  {
    struct {
      const char* name;
      void (*edit)(msa_dims_t*);
      msa_status_t want;
    } cases[] = {
        {"batch 0", [](msa_dims_t* d) { d->batch = 0; }, MSA_ERR_BAD_DIMS},
        {"heads", [](msa_dims_t* d) { d->num_q_heads = 60; }, MSA_ERR_BAD_DIMS},
        {"hpg", [](msa_dims_t* d) { d->num_q_heads = 48; }, MSA_ERR_UNSUPPORTED},
        {"kv heads", [](msa_dims_t* d) { d->num_kv_heads = 65536; d->num_q_heads = 131072; }, MSA_ERR_UNSUPPORTED},
        {"head dim", [](msa_dims_t* d) { d->head_dim = 96; }, MSA_ERR_UNSUPPORTED},
        {"index dim", [](msa_dims_t* d) { d->index_dim = 48; }, MSA_ERR_UNSUPPORTED},
        {"block", [](msa_dims_t* d) { d->block_size = 64; }, MSA_ERR_UNSUPPORTED},
        {"top_k 0", [](msa_dims_t* d) { d->top_k = 0; }, MSA_ERR_BAD_DIMS},
        {"top_k 33", [](msa_dims_t* d) { d->top_k = 33; }, MSA_ERR_BAD_DIMS},
        {"scale", [](msa_dims_t* d) { d->softmax_scale = -1.f; }, MSA_ERR_BAD_DIMS},
        {"scale inf", [](msa_dims_t* d) { d->softmax_scale = 1.f / 0.f; }, MSA_ERR_BAD_DIMS},
        {"total_q > total_k", [](msa_dims_t* d) { d->total_q = 40000; }, MSA_ERR_BAD_DIMS},
        {"negative totals", [](msa_dims_t* d) { d->total_q = -1; }, MSA_ERR_BAD_DIMS},
        {"q 2^26", [](msa_dims_t* d) { d->total_q = 1 << 26; d->total_k = 1 << 27; d->max_q_len = d->max_k_len = 1; }, MSA_ERR_UNSUPPORTED},
        {"k 2^31", [](msa_dims_t* d) { d->total_k = (int64_t)1 << 31; }, MSA_ERR_UNSUPPORTED},
        {"max lens", [](msa_dims_t* d) { d->max_q_len = 40000; }, MSA_ERR_BAD_DIMS},
        {"chunk", [](msa_dims_t* d) { d->q_chunk = -1; }, MSA_ERR_BAD_DIMS},
        {"flags", [](msa_dims_t* d) { d->flags = 2; }, MSA_ERR_BAD_DIMS},
        {"flags all", [](msa_dims_t* d) { d->flags = -1; }, MSA_ERR_BAD_DIMS},
        {"pages no table", [](msa_dims_t* d) { d->kv_pages = 256; }, MSA_ERR_NULL_ARG},
        {"table no pages", [](msa_dims_t* d) { d->block_table = (const int32_t*)64; }, MSA_ERR_BAD_DIMS},
        {"pages mismatch", [](msa_dims_t* d) { d->kv_pages = 255; d->block_table = (const int32_t*)64; d->max_blocks_per_seq = 256; }, MSA_ERR_BAD_DIMS},
        {"pairs 2^24", [](msa_dims_t* d) { d->batch = 65535; d->num_q_heads = 512; d->num_kv_heads = 512; d->total_q = 65535; d->total_k = 1 << 20; d->max_q_len = 1; d->max_k_len = 16; }, MSA_ERR_UNSUPPORTED},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
      msa_dims_t d = base_dims();
      cases[i].edit(&d);
      size_t bytes = 0;
      EXPECT(msa_workspace_size(&d, MSA_OP_ATTEND, &bytes) == cases[i].want, cases[i].name);
      EXPECT(msa_attend_pass_rows(&d) == -(int64_t)cases[i].want, cases[i].name);
    }
    EXPECT(msa_workspace_size(NULL, MSA_OP_ATTEND, NULL) == MSA_ERR_NULL_ARG, "null dims");
    msa_dims_t d = base_dims();
    EXPECT(msa_workspace_size(&d, MSA_OP_ATTEND, NULL) == MSA_ERR_NULL_ARG, "null bytes");
    size_t nb = 0;
    EXPECT(msa_workspace_size(&d, (msa_op_t)9, &nb) == MSA_ERR_BAD_DIMS, "bad op");
  }

  // every entry point: NULL pointers, misalignment and small workspaces are
  // caught on the host (nothing reaches the GPU)
  {
    msa_dims_t d = base_dims();
    static char buf[4096] __attribute__((aligned(256)));
    void* a = buf;                       // aligned stand-in (never dereferenced on failure paths)
    void* m = buf + 1;                   // misaligned
    int32_t* ia = (int32_t*)buf;
    EXPECT(msa_index_select(&d, NULL, a, ia, ia, ia, NULL, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "select null");
    EXPECT(msa_index_select(&d, m, a, ia, ia, ia, NULL, a, 1 << 20, NULL) == MSA_ERR_ALIGNMENT, "select align");
    msa_dims_t dd = base_dims();
    dd.batch = 32; dd.total_q = 32; dd.total_k = 32 * 65536; dd.max_q_len = 1; dd.max_k_len = 65536;
    EXPECT(msa_index_select(&dd, a, a, ia, ia, ia, NULL, a, 16, NULL) == MSA_ERR_WORKSPACE_TOO_SMALL, "select ws");
    EXPECT(msa_build_block_query_lists(&d, ia, NULL, ia, ia, ia, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "lists null");
    EXPECT(msa_build_block_query_lists(&d, ia, ia, ia, ia, ia, a, 16, NULL) == MSA_ERR_WORKSPACE_TOO_SMALL, "lists ws");
    EXPECT(msa_attend(&d, NULL, a, a, ia, ia, ia, ia, ia, a, NULL, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "attend null");
    EXPECT(msa_attend(&d, a, a, a, ia, ia, ia, ia, ia, a, NULL, a, 16, NULL) == MSA_ERR_WORKSPACE_TOO_SMALL, "attend ws");
    EXPECT(msa_attend(&d, a, a, a, ia, ia, ia, ia, ia, m, NULL, a, 1 << 20, NULL) == MSA_ERR_ALIGNMENT, "attend align");
    EXPECT(msa_attend_noalloc(&d, a, a, a, ia, ia, ia, ia, ia, a, NULL, NULL) == MSA_ERR_WORKSPACE_TOO_SMALL, "noalloc size");
    uint8_t* e = (uint8_t*)buf;
    EXPECT(msa_attend_fp8(&d, a, NULL, a, e, a, e, ia, ia, ia, ia, ia, a, NULL, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "fp8 null");
    EXPECT(msa_attend_q8kv4(&d, a, e, a, NULL, a, e, ia, ia, ia, ia, ia, a, NULL, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "q8kv4 null");
    msa_dims_t dc = base_dims();
    dc.flags = MSA_FLAG_COMPACT_PARTIALS;
    EXPECT(msa_attend_with_mass(&dc, a, a, a, ia, ia, ia, ia, ia, a, NULL, (float*)a, a, 1 << 20, NULL) == MSA_ERR_UNSUPPORTED, "mass compact");
    EXPECT(msa_index_select_fp8(&d, a, e, a, e, ia, ia, ia, NULL, NULL, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "fp8 select null");
    EXPECT(msa_index_select_q8k4(&d, a, e, m, e, ia, ia, ia, NULL, a, 1 << 20, NULL) == MSA_ERR_ALIGNMENT, "q8k4 select align");
    EXPECT(msa_index_quantize_fp8(&d, a, a, NULL, a, e, a, e, NULL) == MSA_ERR_NULL_ARG, "quant fp8 null");
    EXPECT(msa_index_quantize_q8k4(&d, m, NULL, ia, a, e, a, e, NULL) == MSA_ERR_ALIGNMENT, "quant q8k4 align");
    EXPECT(msa_main_quantize_fp8(&d, a, a, a, NULL, a, e, a, e, a, e, NULL) == MSA_ERR_NULL_ARG, "main quant null");
    EXPECT(msa_main_quantize_q8kv4(&d, a, a, a, ia, a, e, m, e, a, e, NULL) == MSA_ERR_ALIGNMENT, "main q8kv4 align");
    EXPECT(msa_index_project(&d, 100, a, a, a, ia, ia, a, a, a, 1 << 20, NULL) == MSA_ERR_UNSUPPORTED, "project dim");
    EXPECT(msa_index_project(&d, 4096, NULL, a, a, ia, ia, a, a, a, 1 << 20, NULL) == MSA_ERR_NULL_ARG, "project null");
    EXPECT(msa_index_kl(&d, a, a, ia, ia, ia, NULL, (float*)a, NULL, (float*)a, NULL) == MSA_ERR_NULL_ARG, "kl null");
    EXPECT(msa_hbm_stream(a, 15, 2, a, a, NULL) == MSA_ERR_BAD_DIMS, "stream size");
    EXPECT(msa_hbm_stream(a, 16, 5, a, a, NULL) == MSA_ERR_BAD_DIMS, "stream ratio");
    EXPECT(msa_hbm_stream(m, 16, 1, a, a, NULL) == MSA_ERR_ALIGNMENT, "stream align");
    EXPECT(msa_hbm_stream(a, 16, 1, NULL, a, NULL) == MSA_ERR_NULL_ARG, "stream null");
    float ms[MSA_PROFILE_KERNELS];
    int32_t n[MSA_PROFILE_KERNELS];
    EXPECT(msa_profile_collect(NULL, n) == MSA_ERR_NULL_ARG, "profile null");
    EXPECT(msa_profile_collect(ms, n) == MSA_OK, "profile empty collect");
    for (int i = -1; i <= MSA_PROFILE_KERNELS; ++i) EXPECT(msa_profile_kernel_name(i) != NULL, "kernel name");
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
