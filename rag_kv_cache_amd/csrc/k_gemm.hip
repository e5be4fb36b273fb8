// GEMMs of the fusion step: C[M][N] = A[M][K] * B[N][K]^T (B = nn.Linear weight rows) with a
// fused epilogue.  Used for the fresh K/V and Q of the selected rows (RoPE epilogue), the
// o-projection and the FFN down-projection (residual-add epilogue), and the FFN gate/up
// projection (SwiGLU epilogue).
//
// Logical output columns are the weight rows in their natural order (for SwiGLU: the gate
// rows, then the up rows).  The epilogues combine pairs of logical columns:
//   RoPE   (n, n + head_dim/2) of the same head (rotation by the row's position),
//   SwiGLU (f, ffn + f): silu(gate) * up of feature f,
//   store / residual: independent columns.
//
// bf16 path (v_mfma_f32_16x16x32_bf16, gfx950):
//   * workgroup tile BM x BN x 64 with WM x WN wavefronts, each owning a (BM/WM) x (BN/WN)
//     block of 16x16 MFMA tiles;
//   * operands go global -> LDS directly (global_load_lds_dwordx4, no staging registers) into
//     a 3-stage ring, two K-steps ahead of the MFMAs; one barrier per K-step;
//   * inside each tile the weight rows are permuted in 16-row blocks so that the two
//     columns of every epilogue pair land in adjacent MFMA tiles: the same lane then holds
//     both values and the epilogue runs from registers;
//   * rows of A may be gathered through an index list (the kept rows); rows past M read a
//     clamped row (never stored), so the loads are branch-free;
//   * tiles are assigned XCD-contiguously (xcd_tile) so that the workgroups reading the same
//     weight rows share one XCD's L2;
//   * split-K (grid.y > 1) writes fp32 partials in logical column order; a reduce kernel
//     sums them and applies the same epilogue.
//
// MFMA 16x16x32 operand layout: lane l supplies row (l & 15) of A and column (l & 15) of B,
// both with reduction slots (l >> 4) * 8 .. + 7; lane l receives C[4 * (l >> 4) + r][l & 15].
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

constexpr int BK = 64;

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// Epilogue on one pair of logical columns (n_a, n_b) of row m.
template <int EPI, typename TO>
__device__ __forceinline__ void epi_pair(const GemmArgs& g, int m, int n_a, int n_b, float va, float vb) {
  if (EPI == EPI_ROPE) {
    if (n_a < g.rope_cols) {
      int p = g.pos[m];
      p = p < 0 ? 0 : (p > g.max_pos ? g.max_pos : p);
      const float2 t = g.rope[(long)p * (g.head_dim >> 1) + (n_a % g.head_dim)];
      const float ya = va * t.x - vb * t.y;
      const float yb = vb * t.x + va * t.y;
      va = ya;
      vb = yb;
    }
    TO* o = (TO*)g.out + (long)m * g.ldo;
    Elem<TO>::st(o + n_a, va);
    Elem<TO>::st(o + n_b, vb);
  } else if (EPI == EPI_SWIGLU) {
    TO* o = (TO*)g.out + (long)m * g.ldo;
    Elem<TO>::st(o + n_a, silu(va) * vb);
  } else if (EPI == EPI_RESID) {
    const long rr = g.resid_rows ? (long)g.resid_rows[m] : (long)m;
    const float* r = g.resid + rr * g.ldr;
    float* o = (float*)g.out + (long)m * g.ldo;
    o[n_a] = r[n_a] + va;
    o[n_b] = r[n_b] + vb;
  } else {
    TO* o = (TO*)g.out + (long)m * g.ldo;
    Elem<TO>::st(o + n_a, va);
    Elem<TO>::st(o + n_b, vb);
  }
}

// Logical column of tile-local column tc (0..BN-1) of tile tn, for the bf16 kernel's
// in-tile permutation.  Blocks of 16 columns come in pairs (2q, 2q+1) whose columns pair up.
template <int EPI, int BN>
__device__ __forceinline__ int logical_col(const GemmArgs& g, int tn, int tc) {
  const int b = tc >> 4, j = tc & 15, q = b >> 1, odd = b & 1;
  if (EPI == EPI_ROPE) {  // head_dim 128: block q of a head pairs dims 16q.. with 64 + 16q..
    const int head = (tn * BN + tc) >> 7;
    const int qh = q & 3;
    return head * 128 + (odd ? 64 : 0) + qh * 16 + j;
  }
  if (EPI == EPI_SWIGLU) {  // even blocks gate rows, odd blocks up rows of the same features
    const int f = tn * (BN >> 1) + q * 16 + j;
    return odd ? g.swiglu_ffn + f : f;
  }
  return tn * BN + tc;
}

// Each global_load_lds_dwordx4 wave instruction writes its 64 lanes x 16 bytes contiguously
// (lane l at byte 16 l), i.e. 8 tile rows of 128 bytes; the 16-byte chunks of row r are stored
// XOR-swizzled (chunk c at slot c ^ (r & 7)) so that fragment reads of 8 consecutive rows hit
// disjoint banks.
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int ROWB = BK * 2;                       // 128 bytes per tile row
  constexpr int STAGE_B = (BM + BN) * ROWB;
  constexpr int NSTAGE = 3;
  constexpr int A_INS = BM / 8, B_INS = BN / 8;      // 1 KB wave instructions per tile
  constexpr int A_PW = A_INS / NW, B_PW = B_INS / NW;
  static_assert(FN % 2 == 0 && A_INS % NW == 0 && B_INS % NW == 0, "tile shape");
  extern __shared__ __align__(16) unsigned char smem[];

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  if (tile < 0) return;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM;
  const int k_len = g.K / g.splits;
  const int kb = blockIdx.y * k_len;
  const int nk = k_len / BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const char* A = reinterpret_cast<const char*>(g.A);
  const char* B = reinterpret_cast<const char*>(g.B);
  // this lane's source row / chunk inside each 8-row instruction block
  const int r8 = lane >> 3, slot = lane & 7;
  const int chunk = slot ^ r8;  // (tile row & 7) == r8 because blocks are 8-row aligned
  const char* a_src[A_PW];
  const char* b_src[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 8 + r8;
    int m = m0 + row;
    m = m < g.M ? m : g.M - 1;
    const long grow = g.a_rows ? (long)g.a_rows[m] : (long)m;
    a_src[i] = A + (grow * g.lda + kb + chunk * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < B_PW; ++i) {
    const int row = (wave * B_PW + i) * 8 + r8;
    b_src[i] = B + ((long)logical_col<EPI, BN>(g, tn, row) * g.ldb + kb + chunk * 8) * 2;
  }
  auto issue = [&](int kt, int st) __attribute__((always_inline)) {
    unsigned char* base = smem + st * STAGE_B;
#pragma unroll
    for (int i = 0; i < A_PW; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(a_src[i] + kt * BK * 2), (lvoid_t*)(base + (wave * A_PW + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PW; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(b_src[i] + kt * BK * 2), (lvoid_t*)(base + BM * ROWB + (wave * B_PW + i) * 1024), 16, 0, 0);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets: row (l & 15) of each 16-row block, chunk 4*ks + (l >> 4), swizzled
  const int fr = lane & 15, fc = lane >> 4;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int t = 0; t < nk; ++t) {
    // K-step t's loads are this wave's oldest outstanding ones: allow only K-step t+1's
    if (t + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | (A_PW + B_PW));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    // Plain s_barrier: every wave has waited for its own loads of this stage above, and its
    // reads of the stage being refilled were consumed before it reached here.  (The fence of
    // __syncthreads would also drain the loads still in flight for the next K-step.)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (t + 2 < nk) issue(t + 2, (t + 2) % NSTAGE);
    const unsigned char* sa = smem + (t % NSTAGE) * STAGE_B;
    const unsigned char* sb = sa + BM * ROWB;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = 4 * ks + fc;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + row * ROWB + ((c ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 16 + fr;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + row * ROWB + ((c ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  const int row_base = m0 + wm * WTM + (lane >> 4) * 4;
  float* P = g.partial + (long)blockIdx.y * g.M * g.N;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < FN / 2; ++q) {
      const int tc = wn * WTN + q * 32 + (lane & 15);
      const int n_a = logical_col<EPI, BN>(g, tn, tc);
      const int n_b = logical_col<EPI, BN>(g, tn, tc + 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row_base + i * 16 + r;
        if (m >= g.M) continue;
        const float va = acc[i][2 * q][r], vb = acc[i][2 * q + 1][r];
        if (g.splits > 1) {
          P[(long)m * g.N + n_a] = va;
          P[(long)m * g.N + n_b] = vb;
        } else {
          epi_pair<EPI, bf16_t>(g, m, n_a, n_b, va, vb);
        }
      }
    }
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
  constexpr int lds = 3 * (BM + BN) * BK * 2;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM, BN, WM, WN, EPI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN);
  const int grid_x = 8 * ((tiles + 7) / 8);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI>), dim3(grid_x, g.splits), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

// Sum split-K partials (logical columns) and apply the epilogue.  One thread per column pair.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const long half = g.N / 2;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)g.M * half) return;
  const int m = (int)(idx / half);
  const int j = (int)(idx - (long)m * half);
  int n_a, n_b;
  if (EPI == EPI_ROPE) {
    n_a = (j >> 6) * 128 + (j & 63);
    n_b = n_a + 64;
  } else if (EPI == EPI_SWIGLU) {
    n_a = j;
    n_b = j + g.swiglu_ffn;
  } else {
    n_a = j;
    n_b = j + (int)half;
  }
  const long stride = (long)g.M * g.N;
  const float* p = g.partial + (long)m * g.N;
  float va = 0.f, vb = 0.f;
  for (int s = 0; s < g.splits; ++s) {
    va += p[s * stride + n_a];
    vb += p[s * stride + n_b];
  }
  epi_pair<EPI, bf16_t>(g, m, n_a, n_b, va, vb);
}

// ------------------------------------------------------------------ fp32 path
// Correctness configurations: tile 64 x 128 x 16 on the vector ALUs, each thread 4 rows x 8
// columns, operands through LDS; the C tile is staged in LDS and the epilogue pairs columns
// (c, c + 64) of the tile, with the weight rows mapped so that such a pair is a RoPE pair
// (head_dim 64 or 128) or a (gate, up) pair.
constexpr int FBN = 128;
constexpr int FCP = FBN + 4;

__device__ __forceinline__ long f32_b_row(const GemmArgs& g, int tn, int r) {
  if (g.swiglu_ffn > 0) return r < 64 ? (long)tn * 64 + r : (long)g.swiglu_ffn + (long)tn * 64 + (r - 64);
  return (long)tn * FBN + r;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int FBM = 64, FBK = 16;
  __shared__ __align__(16) float smem[FBM * FCP];  // staged C tile; also holds the A/B tiles
  float* As = smem;                // [FBK][FBM]
  float* Bs = smem + FBK * FBM;    // [FBK][FBN]
  const int tiles_m = (g.M + FBM - 1) / FBM;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * FBM, n0 = tn * FBN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* B = reinterpret_cast<const float*>(g.B);
  float acc[4][8] = {};
  const int ar = tid >> 2, ak = (tid & 3) * 4;
  const int am = m0 + ar;
  const bool a_ok = am < g.M;
  const float* a_src = A + (a_ok ? (g.a_rows ? (long)g.a_rows[am] : (long)am) : 0) * g.lda + ak;
  const int br = tid >> 2, bk = (tid & 3) * 4;
  const float* b_src0 = B + f32_b_row(g, tn, br) * g.ldb + bk;
  const float* b_src1 = B + f32_b_row(g, tn, br + 64) * g.ldb + bk;
  for (int k = 0; k < g.K; k += FBK) {
    const float4 av = a_ok ? *reinterpret_cast<const float4*>(a_src + k) : make_float4(0, 0, 0, 0);
    const float4 b0 = *reinterpret_cast<const float4*>(b_src0 + k);
    const float4 b1 = *reinterpret_cast<const float4*>(b_src1 + k);
    As[(ak + 0) * FBM + ar] = av.x; As[(ak + 1) * FBM + ar] = av.y;
    As[(ak + 2) * FBM + ar] = av.z; As[(ak + 3) * FBM + ar] = av.w;
    Bs[(bk + 0) * FBN + br] = b0.x; Bs[(bk + 1) * FBN + br] = b0.y;
    Bs[(bk + 2) * FBN + br] = b0.z; Bs[(bk + 3) * FBN + br] = b0.w;
    Bs[(bk + 0) * FBN + br + 64] = b1.x; Bs[(bk + 1) * FBN + br + 64] = b1.y;
    Bs[(bk + 2) * FBN + br + 64] = b1.z; Bs[(bk + 3) * FBN + br + 64] = b1.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4*>(As + kk * FBM + ty * 4);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float b = Bs[kk * FBN + tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = fmaf(a[i], b, acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) smem[(ty * 4 + i) * FCP + tx + 16 * j] = acc[i][j];
  __syncthreads();
  const int c = tid & 63;
  int c0 = c, c1 = c + 64;
  if (g.epi == EPI_ROPE) {
    const int half = g.head_dim >> 1;
    const int hb = c / half, i = c - hb * half;
    c0 = hb * g.head_dim + i;
    c1 = c0 + half;
  }
  for (int rr = tid >> 6; rr < FBM; rr += 4) {
    const int m = m0 + rr;
    if (m >= g.M) break;
    const float v0 = smem[rr * FCP + c0], v1 = smem[rr * FCP + c1];
    switch (g.epi) {
      case EPI_ROPE: epi_pair<EPI_ROPE, float>(g, m, n0 + c0, n0 + c1, v0, v1); break;
      case EPI_SWIGLU: epi_pair<EPI_SWIGLU, float>(g, m, tn * 64 + c, 0, v0, v1); break;
      case EPI_RESID: epi_pair<EPI_RESID, float>(g, m, n0 + c0, n0 + c1, v0, v1); break;
      default: epi_pair<EPI_STORE, float>(g, m, n0 + c0, n0 + c1, v0, v1);
    }
  }
}

// ------------------------------------------------------------------ launch
template <int EPI>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  hipError_t e;
  const int cfg = gemm_config(g.M, g.N);
  if (cfg == 0) e = launch_dma<128, 256, 2, 4, EPI>(g, s);
  else if (cfg == 1) e = launch_dma<64, 256, 1, 4, EPI>(g, s);
  else e = launch_dma<128, 128, 2, 2, EPI>(g, s);
  if (e != hipSuccess || g.splits <= 1) return e;
  const long items = (long)g.M * (g.N / 2);
  hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

// 0: 128 x 256 tile, 8 wavefronts (the large GEMMs); 1: 64 x 256, 4 wavefronts (a handful of
// rows); 2: 128 x 128, 4 wavefronts (narrow outputs, usually with split-K).
int gemm_config(int M, int N) {
  if (N % 256 == 0 && M <= 64) return 1;
  if (N % 256 == 0 && ((M + 127) / 128) * (N / 256) >= 200) return 0;
  return 2;
}

int gemm_tiles(int M, int N) {
  switch (gemm_config(M, N)) {
    case 0: return ((M + 127) / 128) * (N / 256);
    case 1: return ((M + 63) / 64) * (N / 256);
    default: return ((M + 127) / 128) * (N / 128);
  }
}

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  switch (g.epi) {
    case EPI_ROPE: return launch_epi<EPI_ROPE>(g, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(g, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(g, s);
    default: return launch_epi<EPI_STORE>(g, s);
  }
}

hipError_t gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int tiles = ((g.M + 63) / 64) * (g.N / FBN);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace cb
