// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cb {

enum Epi { EPI_STORE = 0, EPI_ROPE = 1, EPI_SWIGLU = 2, EPI_RESID = 3 };

// C[M][N] = A[M][K] * B[N][K]^T with fp32 accumulation and a fused epilogue.
struct GemmArgs {
  const void* A; long lda; const int32_t* a_rows;  // A row of GEMM row m = a_rows ? a_rows[m] : m
  int a_rows_total;      // rows of A the a_rows entries may address (0: M)
  const void* B; long ldb;
  int swiglu_ffn;        // >0: tile t's columns 0..63 are B rows t*64.., columns 64..127 rows ffn + t*64..
  int M, N, K, splits;   // N % 128 == 0, K % (64 * splits) == 0
  float* partial;        // [splits][M][N] fp32 when splits > 1
  int epi;               // Epi
  void* out; long ldo;   // STORE/ROPE/SWIGLU: dtype; RESID: fp32
  const int32_t* pos; const float2* rope; int rope_cols, head_dim, max_pos;  // ROPE
  const float* resid; long ldr; const int32_t* resid_rows;                  // RESID
  const float* norm_g; float norm_eps; void* norm_out;  // RESID: also RMSNorm(out) -> bf16 [M][N]
  int cfg;               // bf16 tile configuration (GemmCfg), from gemm_plan
  int b_i8;              // B is int8 [N][ldb] with per-row (output channel) scales bscale[N]
  const float* bscale;
  // skinny product (GEMM_GEMV) only: when a_f32 is set, A row m is RMSNorm(a_f32 row) * a_gain
  // (row a_rows ? a_rows[m] : m, stride lda, K wide), formed as bf16 on load; A is not read
  const float* a_f32; const float* a_gain; float a_eps;
  // ROPE only: when kv_k is set, logical columns kv_col0 .. kv_col0 + 2 kvd - 1 (K, then V) of
  // row m go to row pos[m] of kv_k / kv_v ([kv_rows][kvd]; rows outside are skipped) instead of
  // out, and sel_out[m] = pos[m], local_out[m] = m (every plan: tiles, split-K reduce, skinny)
  void* kv_k; void* kv_v; int kv_col0, kvd, kv_rows; int32_t* sel_out; int32_t* local_out;
};
hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s);
enum GemmCfg { GEMM_128x512 = 0, GEMM_128x256 = 1, GEMM_64x256 = 2, GEMM_128x128 = 3, GEMM_64x128 = 4, GEMM_256x256 = 5, GEMM_GEMV = 6 };
struct GemmPlan { int cfg, splits; };
// Tile configuration and split-K factor of the bf16 GEMM for an M x N x K product with
// epilogue `epi`; split partials ([splits][M][N] fp32) must fit partial_cap_elems.
GemmPlan gemm_plan(int M, int N, int K, int epi, long partial_cap_elems);
hipError_t gemm_f32(const GemmArgs& g, hipStream_t s);

// Causal GQA attention of n_q query rows (positions qpos, ascending) over K/V rows 0..N-1.
struct AttnArgs {
  const void* q; long ldq; const int32_t* qpos; int n_q;
  const void* k; const void* v; int n_tok, hq, hkv, dh;
  void* out; long ldo;
  int splits, split_len;       // key range of split s: [s*split_len, (s+1)*split_len)
  float* part_o; float* part_ml;
  float scale_log2;            // log2(e) / sqrt(head_dim)
};
hipError_t attn_bf16(const AttnArgs& a, hipStream_t s);
// Query rows per workgroup of the bf16 attention for a GQA group of `group` query heads.
int attn_rows_per_wg(int group);
// Whether n_q query rows of a group of `group` heads run on the few-row (decode) kernel, whose
// key ranges may be any multiple of 16 keys (other kernels: multiples of 64), at most 64 ranges.
bool attn_decode_fits(int n_q, int group);
hipError_t attn_f32(const AttnArgs& a, hipStream_t s);

hipError_t embed(const int32_t* tok, int n, const void* table, int vocab, int d, int bf16, float* out,
                 hipStream_t s);
hipError_t rmsnorm(const float* h, long ldh, int n, int d, const float* g, float eps, void* out, int bf16,
                   hipStream_t s);
// Per-layer buffers of a batched position update (at most kRopeMaxLayers per launch).
constexpr int kRopeMaxLayers = 64;
struct RopeLayers {
  const void* kc[kRopeMaxLayers];
  const void* vc[kRopeMaxLayers];
  void* kf[kRopeMaxLayers];
  void* vf[kRopeMaxLayers];
};
// rope_delta for n_layers layers in one launch; copy_v = 0 when every V cache aliases its fused V.
hipError_t rope_delta_layers(const RopeLayers& L, int n_layers, int n_ctx, int hkv, int dh, const int32_t* offs,
                             int n_chunks, const float2* table, int table_rows, int copy_v, int bf16, hipStream_t s);
// One layer's cached rows of up to kFetchMaxChunks chunks in pinned host memory (device-
// accessible addresses): chunk c holds rows [offs[c], offs[c+1]) of the fused buffers.
constexpr int kFetchMaxChunks = 64;
struct FetchChunks {
  const void* hk[kFetchMaxChunks];
  const void* hv[kFetchMaxChunks];
  int offs[kFetchMaxChunks + 1];
  int n;
};
// Launch shape of the fetch: workgroups, threads per workgroup (a multiple of 64, <= 1024) and
// 16-byte row pieces each thread keeps in flight (1, 2 or 4; four loads each).
struct FetchLaunch {
  int blocks, threads, unroll;
};
// Read them, rotate K by R(o_c), copy V, into kf / vf (device).
hipError_t fetch_rope(const FetchChunks& F, void* kf, void* vf, int hkv, int dh, const float2* table, int table_rows,
                      int bf16, const FetchLaunch& fl, hipStream_t s);
// table: [table_rows][dh / 2] cos/sin; a chunk offset outside [0, table_rows) is clamped.
hipError_t rope_delta(const void* kc, const void* vc, void* kf, void* vf, int n_ctx, int hkv, int dh,
                      const int32_t* offs, int n_chunks, const float2* table, int table_rows, int bf16,
                      hipStream_t s);
hipError_t dev_scatter(const void* fresh, long ld_fresh, void* fk, void* fv, const int32_t* sel, int n_sel,
                       int n_cand, int n_tok, int row_elems, float* dev, int32_t* copy_sel, int32_t* copy_local,
                       int cosine, int bf16, hipStream_t s);
hipError_t topk_select(const float* dev, const int32_t* sel, int n_cand, int n_query, int k, int32_t* new_sel,
                       int32_t* new_local, hipStream_t s);

}  // namespace cb
