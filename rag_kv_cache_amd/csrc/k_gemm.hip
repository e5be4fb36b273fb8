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
//   * operands go global -> LDS directly (buffer_load_dwordx4 ... lds, no staging registers) into
//     an NS-stage ring (2 to 4 stages by tile; the 256 x 256 tile up to 4096 rows keeps a third
//     stage of the weight tile in a ring of its own), so the loads run NS - 1 K-steps (the
//     weights' one more) ahead of the MFMAs; one barrier per K-step;
//   * inside each tile the weight rows are permuted in 16-row blocks so that the two
//     columns of every epilogue pair land in adjacent MFMA tiles: the same lane then holds
//     both values and the epilogue runs from registers;
//   * rows of A may be gathered through an index list (the kept rows); rows past M read a
//     clamped row (never stored), so the loads are branch-free;
//   * tiles are assigned XCD-contiguously (xcd_tile) and in bands of 8 M-tiles, so that the
//     workgroups running together on one XCD share their A rows and weight rows in its L2;
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

__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

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
    if (g.kv_k) {  // K/V columns go to the fused rows; the pair (n, n + 64) stays in one head
      if (n_a == 0) {
        g.sel_out[m] = g.pos[m];
        g.local_out[m] = m;
      }
      if (n_a >= g.kv_col0) {
        const int j = g.pos[m];
        if (j < 0 || j >= g.kv_rows) return;
        const int kn = n_a - g.kv_col0;
        TO* d = kn < g.kvd ? (TO*)g.kv_k + (long)j * g.kvd + kn : (TO*)g.kv_v + (long)j * g.kvd + (kn - g.kvd);
        Elem<TO>::st(d, va);
        Elem<TO>::st(d + (n_b - n_a), vb);
        return;
      }
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

// Column of tile-local column tc in the staged output tile: the logical column relative to the
// tile's first one (RoPE tiles hold whole heads); for SwiGLU the gate/up feature index, with up
// columns after the BN/2 gate columns (fp32 staging; the bf16 staging uses the gate index).
template <int EPI, int BN>
__device__ __forceinline__ int stage_col(int tc) {
  const int b = tc >> 4, j = tc & 15, q = b >> 1, odd = b & 1;
  if (EPI == EPI_ROPE) return (tc & ~127) + (odd ? 64 : 0) + (q & 3) * 16 + j;
  if (EPI == EPI_SWIGLU) return (odd ? BN / 2 : 0) + q * 16 + j;
  return tc;
}

// Each buffer_load_dwordx4 ... lds wave instruction writes its 64 lanes x 16 bytes contiguously
// (lane l at byte 16 l), i.e. 8 tile rows of 128 bytes; the 16-byte chunks of row r are stored
// XOR-swizzled (chunk c at slot c ^ (r & 7)) so that fragment reads of 8 consecutive rows hit
// disjoint banks.

// s_waitcnt with only vmcnt (N) or only lgkmcnt (0) constrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Wait until at most `ahead` K-steps of LPW load instructions each are still in flight (the
// count saturates at the counter's limit of 63, which only waits longer).
template <int N>
struct Sat63 { static constexpr int v = N < 63 ? N : 63; };
template <int LPW>
__device__ __forceinline__ void wait_vm_steps(int ahead) {
  switch (ahead <= 0 ? 0 : (ahead > 7 ? 7 : ahead)) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<Sat63<LPW>::v>(); break;
    case 2: wait_vm<Sat63<2 * LPW>::v>(); break;
    case 3: wait_vm<Sat63<3 * LPW>::v>(); break;
    case 4: wait_vm<Sat63<4 * LPW>::v>(); break;
    case 5: wait_vm<Sat63<5 * LPW>::v>(); break;
    case 6: wait_vm<Sat63<6 * LPW>::v>(); break;
    default: wait_vm<Sat63<7 * LPW>::v>(); break;
  }
}

// amdgpu_waves_per_eu(2): a register budget of 256 arch VGPRs; with more, the 4-wave tiles
// get their accumulators in AGPRs and copy them around in the main loop.
// Eight int8 weights (two dwords) as eight bf16 (exact for |q| <= 127) in a 16-byte chunk.
__device__ __forceinline__ uint4 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  float f[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f[b] = (float)(int8_t)(lo >> (8 * b));
    f[4 + b] = (float)(int8_t)(hi >> (8 * b));
  }
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// Row halves in which an fp32 output tile is staged: two when the whole tile (BM rows of BN
// fp32 + 16 bytes) exceeds the 160 KiB of LDS.
template <int BM, int BN>
constexpr int gemm_f32_halves() {
  return BM * (BN * 4 + 16) > 160 * 1024 ? 2 : 1;
}

// BT = 0: bf16 weights, global -> LDS by DMA like the activations.  BT = 1: int8 weights with a
// per-output-channel scale (g.bscale): a K-step's weight tile goes global -> registers one
// K-step ahead, is converted to bf16 (exact) and written to the same LDS layout, so the MFMA
// loop is unchanged; the scale multiplies the fp32 sums before the epilogue (split-K: in the
// reduce).
template <int BM, int BN, int WM, int WN, int NS, int EPI, int BT, int XB = 0>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2))) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int ROWB = BK * 2;                       // 128 bytes per tile row
  constexpr int STAGE_B = (BM + BN) * ROWB;
  constexpr int A_INS = BM / 8, B_INS = BN / 8;      // 1 KB wave instructions per tile
  constexpr int A_PW = A_INS / NW, B_PW = B_INS / NW;
  constexpr int LPW = A_PW + B_PW;                   // load instructions per wave per K-step
  static_assert(FN % 2 == 0 && A_INS % NW == 0 && B_INS % NW == 0, "tile shape");
  static_assert(NS >= 2 && NS <= 8, "stages");
  static_assert(XB == 0 || (XB >= 1 && XB <= 4 && BT == 0), "a deeper weight ring: bf16 weights only");
  extern __shared__ __align__(16) unsigned char smem[];

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = g.N / BN;
  const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  if (tile < 0) return;
  // grouped order: bands of up to 8 M-tiles, M fastest inside a band, so that the workgroups
  // running together on one XCD share both their A row blocks and their weight blocks in L2
  constexpr int GM = 8;
  const int band = tile / (GM * tiles_n);
  const int bm0 = band * GM;
  const int bh = min(GM, tiles_m - bm0);
  const int in_band = tile - band * GM * tiles_n;
  const int tm = bm0 + in_band % bh, tn = in_band / bh;
  const int m0 = tm * BM;
  // K-steps of this split: an even share of the K / 64 steps (shares differ by at most one)
  const int nk_all = g.K / BK;
  const int kb0 = (int)((long)nk_all * blockIdx.y / g.splits);
  const int nk = (int)((long)nk_all * (blockIdx.y + 1) / g.splits) - kb0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // the same value, in a scalar register
  // this lane's source row / chunk inside each 8-row instruction block; byte offsets from the
  // operand bases (below 2 GiB: checked at launch), advanced per K-step by a scalar offset
  const int r8 = lane >> 3, slot = lane & 7;
  const int chunk = slot ^ r8;  // (tile row & 7) == r8 because blocks are 8-row aligned
  const int a_bytes = (int)((long)(g.a_rows_total ? g.a_rows_total : g.M) * g.lda * 2);
  const int b_bytes = (int)((long)g.N * g.ldb * 2);
  uint32_t a_vo[A_PW], b_vo[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 8 + r8;
    int m = m0 + row;
    m = m < g.M ? m : g.M - 1;
    const long grow = g.a_rows ? (long)g.a_rows[m] : (long)m;
    a_vo[i] = (uint32_t)((grow * g.lda + (long)kb0 * BK + chunk * 8) * 2);
  }
  if constexpr (BT == 0) {
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
      const int row = (wave * B_PW + i) * 8 + r8;
      b_vo[i] = (uint32_t)(((long)logical_col<EPI, BN>(g, tn, row) * g.ldb + (long)kb0 * BK + chunk * 8) * 2);
    }
  }
  // int8 weights: thread tid owns 16-byte pieces ci = tid + j * threads of the tile's 64-byte
  // K-step rows (row ci / 4, piece ci % 4), i.e. bf16 chunks 2 (ci % 4) and 2 (ci % 4) + 1
  constexpr int CPT = BT ? BN * 4 / (64 * NW) : 1;
  static_assert(!BT || (BN * 4) % (64 * NW) == 0, "int8 weight pieces per thread");
  long b8_off[CPT];
  int b8_lds[CPT];
  uint4 rb[CPT];
  if constexpr (BT) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ci = tid + j * 64 * NW;
      const int row = ci >> 2, pc = ci & 3;
      b8_off[j] = (long)logical_col<EPI, BN>(g, tn, row) * g.ldb + (long)kb0 * BK + pc * 16;
      b8_lds[j] = BM * ROWB + row * ROWB;
      rb[j] = make_uint4(0, 0, 0, 0);
    }
  }
  auto load_b8 = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) rb[j] = *reinterpret_cast<const uint4*>((const char*)g.B + b8_off[j] + (long)kt * BK);
  };
  auto store_b8 = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ci = tid + j * 64 * NW;
      const int row = ci >> 2, pc = ci & 3;
      unsigned char* rp = smem + st * STAGE_B + b8_lds[j];
      *reinterpret_cast<uint4*>(rp + (((2 * pc) ^ (row & 7)) << 4)) = i8x8_to_bf16(rb[j].x, rb[j].y);
      *reinterpret_cast<uint4*>(rp + (((2 * pc + 1) ^ (row & 7)) << 4)) = i8x8_to_bf16(rb[j].z, rb[j].w);
    }
  };
  auto issue = [&](int kt, int st) __attribute__((always_inline)) {
    unsigned char* base = smem + st * STAGE_B;
    const int koff = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < A_PW; ++i) buffer_load_lds16(g.A, a_bytes, base + (wv * A_PW + i) * 1024, a_vo[i], koff);
    if constexpr (BT == 0) {
#pragma unroll
      for (int i = 0; i < B_PW; ++i)
        buffer_load_lds16(g.B, b_bytes, base + BM * ROWB + (wv * B_PW + i) * 1024, b_vo[i], koff);
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment reads: row (l & 15) of each 16-row block, 16-byte chunk 4*ks + (l >> 4) (swizzled).
  // Block rows are multiples of 16, so the swizzle term depends on the lane only.
  const int fr = lane & 15, fc = lane >> 4;
  const int a_off = (wm * WTM + fr) * ROWB, b_off = BM * ROWB + (wn * WTN + fr) * ROWB;
  const int sw0 = ((fc) ^ (fr & 7)) << 4, sw1 = ((4 + fc) ^ (fr & 7)) << 4;
  auto read = [&](int st, int ks, bf16x8_t (&af)[FM], bf16x8_t (&bfr)[FN]) __attribute__((always_inline)) {
    const unsigned char* s = smem + st * STAGE_B + (ks ? sw1 : sw0);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(s + a_off + i * 16 * ROWB);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(s + b_off + j * 16 * ROWB);
  };
  auto mma = [&](const bf16x8_t (&af)[FM], const bf16x8_t (&bfr)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // Pipeline: K-steps t .. t+NS-1 occupy the NS stages; fragments of the two 32-wide halves of
  // a K-step are double-buffered in registers, so the LDS reads of one half overlap the MFMAs
  // of the other.  At the one barrier per K-step every wave has (a) waited for its own loads of
  // K-step t+1 and (b) finished reading stage t, which is then refilled with K-step t+NS.  The
  // steady loop has a constant wait and no branch; the last NS-1 K-steps drain separately.
  // int8 weights: the tile of K-step t+NS is loaded into registers after the barrier of
  // iteration t (before that step's DMA, so that one wait leaves only the DMA in flight) and
  // written to its stage, converted, in iteration t+1 before that iteration's barrier; the
  // stage was read for the last time before iteration t's barrier and is next read in
  // iteration t+NS > t+1.
  constexpr int LPWD = BT ? A_PW : LPW;  // DMA instructions per wave per K-step
  if constexpr (XB == 1) {
    // A deeper weight ring: NS stages of the activation tile, NS + XB of the weight tile, in
    // two separate rings (activations first, then weights).  Weight K-step t + NS + XB is
    // issued in iteration t, after the activation K-step t + NS, so each weight load gets XB
    // more iterations to land; the wait before the barrier of iteration t must see the
    // activations of K-step t + 1 (issued in iteration t + 1 - NS): what was issued after them
    // may still be in flight, i.e. that iteration's weights and the NS - 2 later iterations'
    // loads (the weights of K-step t + 1 were issued XB iterations before its activations).
    constexpr int NSB = NS + XB;
    constexpr int SA_B = BM * ROWB, SB_B = BN * ROWB;
    unsigned char* const ra = smem;
    unsigned char* const rbw = smem + NS * SA_B;
    auto issue_a = [&](int kt, int sa) __attribute__((always_inline)) {
      unsigned char* base = ra + sa * SA_B;
#pragma unroll
      for (int i = 0; i < A_PW; ++i) buffer_load_lds16(g.A, a_bytes, base + (wv * A_PW + i) * 1024, a_vo[i], kt * BK * 2);
    };
    auto issue_b = [&](int kt, int sb) __attribute__((always_inline)) {
      unsigned char* base = rbw + sb * SB_B;
#pragma unroll
      for (int i = 0; i < B_PW; ++i) buffer_load_lds16(g.B, b_bytes, base + (wv * B_PW + i) * 1024, b_vo[i], kt * BK * 2);
    };
    const int b_roff = (wn * WTN + fr) * ROWB;  // fragment row of the weight tile within a stage
    auto readx = [&](int sa, int sb, int ks, bf16x8_t (&af)[FM], bf16x8_t (&bfr)[FN]) __attribute__((always_inline)) {
      const unsigned char* pa = ra + sa * SA_B + (ks ? sw1 : sw0);
      const unsigned char* pb = rbw + sb * SB_B + (ks ? sw1 : sw0);
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(pa + a_off + i * 16 * ROWB);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(pb + b_roff + j * 16 * ROWB);
    };
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      if (s < NS && s < nk) issue_a(s, s);
      if (s < nk) issue_b(s, s);
    }
    wait_vm<0>();
    barrier();
    bf16x8_t a0[FM], b0[FN], a1[FM], b1[FN];
    readx(0, 0, 0, a0, b0);
    int sa = 0, sb = 0, t = 0;
    for (; t + NSB < nk; ++t) {
      readx(sa, sb, 1, a1, b1);
      mma(a0, b0);
      wait_lgkm0();
      wait_vm<Sat63<B_PW + (NS - 2) * LPW>::v>();  // K-step t+1 landed
      barrier();
      issue_a(t + NS, sa);
      issue_b(t + NSB, sb);
      sa = sa + 1 == NS ? 0 : sa + 1;
      sb = sb + 1 == NSB ? 0 : sb + 1;
      readx(sa, sb, 0, a0, b0);
      mma(a1, b1);
    }
    for (; t + 1 < nk; ++t) {  // the last NS K-steps: refill what remains, wait for everything
      readx(sa, sb, 1, a1, b1);
      mma(a0, b0);
      wait_lgkm0();
      wait_vm<0>();
      barrier();
      if (t + NS < nk) issue_a(t + NS, sa);
      if (t + NSB < nk) issue_b(t + NSB, sb);
      sa = sa + 1 == NS ? 0 : sa + 1;
      sb = sb + 1 == NSB ? 0 : sb + 1;
      readx(sa, sb, 0, a0, b0);
      mma(a1, b1);
    }
    readx(sa, sb, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  } else {
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nk) issue(s, s);
  if constexpr (BT == 0) {
    wait_vm_steps<LPW>(min(NS - 1, nk - 1));  // K-step 0 landed; later K-steps may be in flight
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) {  // the first stages' weights, one stage at a time
      if (s < nk) {
        load_b8(s);
        wait_vm<0>();
        store_b8(s);
      }
    }
    wait_lgkm0();
  }
  barrier();
  bf16x8_t a0[FM], b0[FN], a1[FM], b1[FN];
  read(0, 0, a0, b0);
  int st = 0, t = 0;
  int pst = -1;  // stage whose int8 weights wait in registers (none: -1)
  for (; t + NS < nk; ++t) {
    read(st, 1, a1, b1);
    mma(a0, b0);
    if constexpr (BT) {
      if (pst >= 0) {
        wait_vm<Sat63<A_PW>::v>();  // only the last K-step's DMA may still be in flight
        store_b8(pst);
      }
    }
    wait_lgkm0();                         // this wave is done reading stage st
    wait_vm<Sat63<(NS - 2) * LPWD>::v>();  // K-step t+1 landed (t+2 .. t+NS-1 may be in flight)
    barrier();
    if constexpr (BT) {
      load_b8(t + NS);
      pst = st;
    }
    issue(t + NS, st);
    st = st + 1 == NS ? 0 : st + 1;
    read(st, 0, a0, b0);
    mma(a1, b1);
  }
  for (; t + 1 < nk; ++t) {
    read(st, 1, a1, b1);
    mma(a0, b0);
    if constexpr (BT) {
      if (pst >= 0) {
        wait_vm<Sat63<A_PW>::v>();
        store_b8(pst);
        pst = -1;
      }
    }
    wait_lgkm0();
    wait_vm_steps<LPWD>(nk - 2 - t);  // K-step t+1 landed
    barrier();
    st = st + 1 == NS ? 0 : st + 1;
    read(st, 0, a0, b0);
    mma(a1, b1);
  }
  read(st, 1, a1, b1);
  mma(a0, b0);
  mma(a1, b1);
  }
  if constexpr (BT) {  // per-output-channel weight scales (split-K partials stay unscaled)
    if (g.splits == 1) {
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int tc = wn * WTN + q * 32 + (lane & 15);
        const float sa = g.bscale[logical_col<EPI, BN>(g, tn, tc)];
        const float sb = g.bscale[logical_col<EPI, BN>(g, tn, tc + 16)];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[i][2 * q][r] *= sa;
            acc[i][2 * q + 1][r] *= sb;
          }
      }
    }
  }

  // Epilogue.  The pair math (RoPE rotation, SwiGLU) runs on the fp32 accumulators in
  // registers; the results are staged in LDS (the operand stages are free by now) in output
  // order and written out along rows with 16-byte stores.  Split-K partials and the residual
  // epilogue stage fp32 values.
  wait_lgkm0();
  barrier();
  const int rl_base = wm * WTM + (lane >> 4) * 4;  // tile row of acc[i][.][0] is rl_base + 16 i
  if (g.splits > 1 || EPI == EPI_RESID) {
    // fp32 tiles too large for LDS (256 x 256: 260 KiB) are staged and written in row halves,
    // each half by the waves whose accumulator rows lie in it
    constexpr int PF = BN * 4 + 16;  // fp32 staging row pitch (bytes)
    constexpr int HALVES = gemm_f32_halves<BM, BN>();
    constexpr int HR = BM / HALVES;  // tile rows per half
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      if (hf > 0) barrier();  // the previous half's reads of the staging rows are done
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          const int tc = wn * WTN + q * 32 + (lane & 15);
          const int la = stage_col<EPI, BN>(tc), lb = stage_col<EPI, BN>(tc + 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = rl_base + i * 16 + r - hf * HR;
            if (HALVES > 1 && (rl < 0 || rl >= HR)) continue;
            unsigned char* row = smem + rl * PF;
            *reinterpret_cast<float*>(row + la * 4) = acc[i][2 * q][r];
            *reinterpret_cast<float*>(row + lb * 4) = acc[i][2 * q + 1][r];
          }
        }
      barrier();
      constexpr int CPR = BN / 4;  // 16-byte chunks per row
      for (int it = tid; it < HR * CPR; it += 64 * NW) {
        const int rl = it / CPR, c = (it - rl * CPR) * 4;
        const int m = m0 + hf * HR + rl;
        if (m >= g.M) continue;
        const float4 v = *reinterpret_cast<const float4*>(smem + rl * PF + c * 4);
        if (g.splits > 1) {
          int n;
          if (EPI == EPI_SWIGLU) n = c < BN / 2 ? tn * (BN / 2) + c : g.swiglu_ffn + tn * (BN / 2) + (c - BN / 2);
          else n = tn * BN + c;
          *reinterpret_cast<float4*>(g.partial + ((long)blockIdx.y * g.M + m) * g.N + n) = v;
        } else {
          const long rr = g.resid_rows ? (long)g.resid_rows[m] : (long)m;
          const float4 r4 = *reinterpret_cast<const float4*>(g.resid + rr * g.ldr + tn * BN + c);
          *reinterpret_cast<float4*>((float*)g.out + (long)m * g.ldo + tn * BN + c) =
              make_float4(r4.x + v.x, r4.y + v.y, r4.z + v.z, r4.w + v.w);
        }
      }
    }
  } else {
    constexpr int OW = EPI == EPI_SWIGLU ? BN / 2 : BN;  // output columns of the tile
    constexpr int PB = OW * 2 + 16;                      // bf16 staging row pitch (bytes)
    // RoPE: positions of this lane's rows up front; the cos/sin of its column pairs (heads are
    // 128 wide on the bf16 path; a pair's first column is dim < 64 of its head) one 16-row block
    // ahead of their use, in two register sets, so that the loads overlap the rotation of the
    // previous block without holding the whole tile's factors at once.
    constexpr int NR = EPI == EPI_ROPE ? FM * 4 : 1, NP = EPI == EPI_ROPE ? (FN / 2) * 4 : 1;
    int prow[NR];
    float2 cs[2][NP];
    auto load_cs = [&](int i, float2 (&c)[NP]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int n_a = logical_col<EPI, BN>(g, tn, wn * WTN + q * 32 + (lane & 15));
#pragma unroll
        for (int r = 0; r < 4; ++r) c[q * 4 + r] = g.rope[prow[i * 4 + r] + (n_a & 127)];
      }
    };
    if (EPI == EPI_ROPE) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int m = m0 + rl_base + i * 16 + r;
          m = m < g.M ? m : g.M - 1;
          const int p = g.pos[m];
          prow[i * 4 + r] = (p < 0 ? 0 : (p > g.max_pos ? g.max_pos : p)) * 64;
        }
      load_cs(0, cs[0]);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (EPI == EPI_ROPE && i + 1 < FM) load_cs(i + 1, cs[(i + 1) & 1]);
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int tc = wn * WTN + q * 32 + (lane & 15);
        const int la = stage_col<EPI, BN>(tc), lb = stage_col<EPI, BN>(tc + 16);
        const bool rot = EPI == EPI_ROPE && logical_col<EPI, BN>(g, tn, tc) < g.rope_cols;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = rl_base + i * 16 + r;
          float va = acc[i][2 * q][r], vb = acc[i][2 * q + 1][r];
          unsigned char* row = smem + rl * PB;
          if (EPI == EPI_SWIGLU) {
            *reinterpret_cast<bf16_t*>(row + la * 2) = f32_to_bf16(silu(va) * vb);
          } else {
            if (rot) {
              const float2 t = cs[i & 1][q * 4 + r];
              const float ya = va * t.x - vb * t.y;
              vb = vb * t.x + va * t.y;
              va = ya;
            }
            *reinterpret_cast<bf16_t*>(row + la * 2) = f32_to_bf16(va);
            *reinterpret_cast<bf16_t*>(row + lb * 2) = f32_to_bf16(vb);
          }
        }
      }
      if (EPI == EPI_ROPE) __builtin_amdgcn_sched_barrier(0);  // keep the next block's loads here
    }
    barrier();
    constexpr int CPR = OW / 8;
    const int colbase = EPI == EPI_SWIGLU ? tn * (BN / 2) : tn * BN;
    for (int it = tid; it < BM * CPR; it += 64 * NW) {
      const int rl = it / CPR, c = (it - rl * CPR) * 8;
      const int m = m0 + rl;
      if (m >= g.M) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(smem + rl * PB + c * 2);
      const int n = colbase + c;
      if (EPI == EPI_ROPE && g.kv_k) {  // K/V columns scattered to the fused rows (8 never straddle K | V)
        if (n == 0) {
          g.sel_out[m] = g.pos[m];
          g.local_out[m] = m;
        }
        if (n >= g.kv_col0) {
          const int j = g.pos[m];
          if (j < 0 || j >= g.kv_rows) continue;
          const int kn = n - g.kv_col0;
          bf16_t* dst = kn < g.kvd ? (bf16_t*)g.kv_k + (long)j * g.kvd + kn : (bf16_t*)g.kv_v + (long)j * g.kvd + (kn - g.kvd);
          *reinterpret_cast<uint4*>(dst) = v;
          continue;
        }
      }
      *reinterpret_cast<uint4*>((bf16_t*)g.out + (long)m * g.ldo + n) = v;
    }
  }
}

// LDS bytes one launch needs: the operand ring, or the staged output tile if larger (an fp32
// tile in row halves when whole it would exceed the LDS).
template <int BM, int BN, int NS, int EPI, int XB = 0>
constexpr int gemm_lds_bytes(bool f32_out) {
  constexpr int ring = NS * (BM + BN) * BK * 2 + XB * BN * BK * 2;
  const int stage = f32_out ? (BM / gemm_f32_halves<BM, BN>()) * (BN * 4 + 16)
                            : BM * ((EPI == EPI_SWIGLU ? BN / 2 : BN) * 2 + 16);
  return ring > stage ? ring : stage;
}

template <int BM, int BN, int WM, int WN, int NS, int EPI, int BT, int XB = 0>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
  constexpr int kMaxLds = 160 * 1024;
  static_assert(NS * (BM + BN) * BK * 2 + XB * BN * BK * 2 <= kMaxLds, "LDS");
  const int lds = gemm_lds_bytes<BM, BN, NS, EPI, XB>(g.splits > 1 || EPI == EPI_RESID);
  if (lds > kMaxLds || g.N % BN != 0 || g.splits < 1 || g.splits > g.K / BK) return hipErrorInvalidValue;
  // operand byte offsets are 32-bit buffer offsets
  const long a_rows = g.a_rows_total ? g.a_rows_total : g.M;
  if (a_rows * g.lda * 2 >= (1L << 31) || (long)g.N * g.ldb * (BT ? 1 : 2) >= (1L << 31)) return hipErrorInvalidValue;
  if (BT && (!g.bscale || g.ldb % 16 != 0)) return hipErrorInvalidValue;
  // once per process (a function-local static is initialised once, also under concurrent calls)
  static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM, BN, WM, WN, NS, EPI, BT, XB>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
  if (attr != hipSuccess) return attr;
  const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN);
  const int grid_x = 8 * ((tiles + 7) / 8);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, NS, EPI, BT, XB>), dim3(grid_x, g.splits), dim3(64 * WM * WN), lds, s, g);
  return hipGetLastError();
}

// Sum split-K partials (logical columns, in split order) and apply the epilogue: one thread
// per 4 consecutive column pairs.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const long half = g.N / 2;
  const long idx = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
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
  float4 va = *reinterpret_cast<const float4*>(p + n_a), vb = *reinterpret_cast<const float4*>(p + n_b);
  for (int s = 1; s < g.splits; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(p + s * stride + n_a);
    const float4 b = *reinterpret_cast<const float4*>(p + s * stride + n_b);
    va.x += a.x; va.y += a.y; va.z += a.z; va.w += a.w;
    vb.x += b.x; vb.y += b.y; vb.z += b.z; vb.w += b.w;
  }
  if (g.bscale) {  // int8 weights: per-output-channel scale of the summed partials
    const float4 sa = *reinterpret_cast<const float4*>(g.bscale + n_a), sb = *reinterpret_cast<const float4*>(g.bscale + n_b);
    va.x *= sa.x; va.y *= sa.y; va.z *= sa.z; va.w *= sa.w;
    vb.x *= sb.x; vb.y *= sb.y; vb.z *= sb.z; vb.w *= sb.w;
  }
  epi_pair<EPI, bf16_t>(g, m, n_a + 0, n_b + 0, va.x, vb.x);
  epi_pair<EPI, bf16_t>(g, m, n_a + 1, n_b + 1, va.y, vb.y);
  epi_pair<EPI, bf16_t>(g, m, n_a + 2, n_b + 2, va.z, vb.z);
  epi_pair<EPI, bf16_t>(g, m, n_a + 3, n_b + 3, va.w, vb.w);
}

// Residual epilogue of a split-K GEMM, one workgroup per output row and one wavefront per
// 256-column block (blocks k = wave, wave + waves, ...):
//   out[m] = resid[resid_rows[m]] + sum_s partial[s][m]   (fp32, split order fixed)
// with every split's partial of a block loaded at once, and, when norm_out is set, the RMSNorm
// of that row (the next GEMM's bf16 A operand) with the same arithmetic as the stand-alone
// RMSNorm kernel: lane l's sum of squares adds blocks k = 0, 1, ... in increasing k (gathered
// through LDS), then the same butterfly.
constexpr int kResidMaxBlocks = 64;   // N <= 16384
constexpr int kResidWavesMax = 8;
__global__ __launch_bounds__(64 * kResidWavesMax) void splitk_resid_norm_kernel(GemmArgs g) {
  __shared__ float sq[kResidMaxBlocks][64];
  constexpr int KW = kResidMaxBlocks / kResidWavesMax;  // blocks per wave kept in registers
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nb = (g.N + 255) / 256;
  const long stride = (long)g.M * g.N;
  const float* p = g.partial + (long)m * g.N;
  const long rr = g.resid_rows ? (long)g.resid_rows[m] : (long)m;
  const float* r = g.resid + rr * g.ldr;
  float* o = (float*)g.out + (long)m * g.ldo;
  float4 w[KW];
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const int k = wave + j * nw;
    if (k >= nb) break;
    const int e = k * 256 + lane * 4;
    float q = 0.f;
    if (e < g.N) {
      float4 a[8];
#pragma unroll
      for (int sp = 0; sp < 8; ++sp)
        if (sp < g.splits) a[sp] = *reinterpret_cast<const float4*>(p + sp * stride + e);
      const float4 rv = *reinterpret_cast<const float4*>(r + e);
      float4 v = a[0];
#pragma unroll
      for (int sp = 1; sp < 8; ++sp)
        if (sp < g.splits) { v.x += a[sp].x; v.y += a[sp].y; v.z += a[sp].z; v.w += a[sp].w; }
      if (g.bscale) {  // int8 weights: per-output-channel scale of the summed partials
        const float4 sc = *reinterpret_cast<const float4*>(g.bscale + e);
        v.x *= sc.x; v.y *= sc.y; v.z *= sc.z; v.w *= sc.w;
      }
      w[j] = make_float4(rv.x + v.x, rv.y + v.y, rv.z + v.z, rv.w + v.w);
      *reinterpret_cast<float4*>(o + e) = w[j];
      q = w[j].x * w[j].x + w[j].y * w[j].y + w[j].z * w[j].z + w[j].w * w[j].w;
    }
    sq[k][lane] = q;
  }
  if (!g.norm_out) return;
  __syncthreads();
  float ss = 0.f;
  for (int k = 0; k < nb; ++k) {
    if (k * 256 + lane * 4 < g.N) ss += sq[k][lane];
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)g.N + g.norm_eps);
  bf16_t* x = (bf16_t*)g.norm_out + (long)m * g.N;
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const int k = wave + j * nw;
    if (k >= nb) break;
    const int e = k * 256 + lane * 4;
    if (e < g.N) {
      const float4 gg = *reinterpret_cast<const float4*>(g.norm_g + e);
      *reinterpret_cast<uint2*>(x + e) =
          make_uint2((uint32_t)f32_to_bf16(w[j].x * rs * gg.x) | ((uint32_t)f32_to_bf16(w[j].y * rs * gg.y) << 16),
                     (uint32_t)f32_to_bf16(w[j].z * rs * gg.z) | ((uint32_t)f32_to_bf16(w[j].w * rs * gg.w) << 16));
    }
  }
}

// Workgroup size of splitk_resid_norm_kernel for N columns.
inline int resid_norm_threads(int N) {
  const int nb = (N + 255) / 256;
  return 64 * (nb < kResidWavesMax ? nb : kResidWavesMax);
}

// ------------------------------------------------------------------ skinny products
// M <= 4 rows (a decode step): weight streaming, not MFMA, bounds the product.  A workgroup of
// four wavefronts owns GV_P epilogue column pairs (2 GV_P weight rows) and splits K in four;
// lane l of a wavefront takes the 16-byte chunks l, l + 64, ... of its K range and keeps fp32
// dot products of every A row with every weight row; the wavefront sums its lanes, the four
// partial sums are added in wavefront order through LDS, and one thread per (row, pair) applies
// the same pair epilogue as the split-K reduce.
constexpr int GV_P = 4;

__device__ __forceinline__ void gv_pair_cols(const GemmArgs& g, int epi, int j, int& n_a, int& n_b) {
  if (epi == EPI_ROPE) {
    n_a = (j >> 6) * 128 + (j & 63);
    n_b = n_a + 64;
  } else if (epi == EPI_SWIGLU) {
    n_a = j;
    n_b = j + g.swiglu_ffn;
  } else {
    n_a = j;
    n_b = j + g.N / 2;
  }
}

__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 w) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(wv[i] << 16), s);
    s = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(wv[i] & 0xffff0000u), s);
  }
  return s;
}

// Dot product of 8 bf16 activations with 8 int8 weights (two dwords).
__device__ __forceinline__ float dot8_bf16_i8(const uint4 a, uint32_t wlo, uint32_t whi) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? wlo : whi;
    const int sh = (i & 1) * 16;
    s = fmaf(__uint_as_float(av[i] << 16), (float)(int8_t)(w >> sh), s);
    s = fmaf(__uint_as_float(av[i] & 0xffff0000u), (float)(int8_t)(w >> (sh + 8)), s);
  }
  return s;
}

// NORM: the activation rows are RMSNorm(g.a_f32 rows) * g.a_gain, formed on load: every
// workgroup first reduces the squares of its MR rows (K floats each, from L2), then scales and
// rounds each 8-element piece to bf16 as it streams K, so no separate normalisation launch is
// needed (measured against staging the rows in LDS first, which delays the weight stream).
template <int EPI, int MR, int BT, int NORM>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(GemmArgs g) {
  constexpr int NR = 2 * GV_P;  // weight rows of the workgroup
  __shared__ float part[4][MR][NR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = blockIdx.x * GV_P;
  const int n_pairs = g.N / 2;
  const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
  const char* B = reinterpret_cast<const char*>(g.B);
  constexpr int WB = BT ? 1 : 2;  // bytes per weight
  const char* wrow[NR];
#pragma unroll
  for (int q = 0; q < GV_P; ++q) {
    int n_a, n_b;
    gv_pair_cols(g, EPI, min(j0 + q, n_pairs - 1), n_a, n_b);
    wrow[2 * q] = B + (long)n_a * g.ldb * WB;
    wrow[2 * q + 1] = B + (long)n_b * g.ldb * WB;
  }
  const bf16_t* arow[MR];
  const float* hrow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int mm = m < g.M ? m : g.M - 1;
    const long r = g.a_rows ? (long)g.a_rows[mm] : (long)mm;
    arow[m] = NORM ? nullptr : A + r * g.lda;
    hrow[m] = NORM ? g.a_f32 + r * g.lda : nullptr;
  }
  float inv[MR];
  if constexpr (NORM) {  // 1 / sqrt(mean of squares + eps) of each row
    __shared__ float red[4][MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float ss = 0.f;
      for (int k = threadIdx.x * 4; k < g.K; k += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(hrow[m] + k);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      if (lane == 0) red[wave][m] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m)
      inv[m] = 1.0f / sqrtf((red[0][m] + red[1][m] + red[2][m] + red[3][m]) / (float)g.K + g.a_eps);
  }
  // this lane's 8 activations at k: read as bf16, or (NORM) h * inv * gain rounded to bf16
  auto load_a = [&](int m, int k) __attribute__((always_inline)) -> uint4 {
    if constexpr (NORM) {
      const float4 h0 = *reinterpret_cast<const float4*>(hrow[m] + k);
      const float4 h1 = *reinterpret_cast<const float4*>(hrow[m] + k + 4);
      const float4 g0 = *reinterpret_cast<const float4*>(g.a_gain + k);
      const float4 g1 = *reinterpret_cast<const float4*>(g.a_gain + k + 4);
      const float r = inv[m];
      return make_uint4(pack_bf16x2(h0.x * r * g0.x, h0.y * r * g0.y), pack_bf16x2(h0.z * r * g0.z, h0.w * r * g0.w),
                        pack_bf16x2(h1.x * r * g1.x, h1.y * r * g1.y), pack_bf16x2(h1.z * r * g1.z, h1.w * r * g1.w));
    } else {
      return *reinterpret_cast<const uint4*>(arow[m] + k);
    }
  };
  const int kq = g.K / 4;  // this wavefront's K range: [wave * kq, (wave + 1) * kq)
  float acc[MR][NR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[m][r] = 0.f;
  for (int k = wave * kq + lane * 8; k < (wave + 1) * kq; k += 512) {
    uint4 a[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) a[m] = load_a(m, k);
    if constexpr (BT) {
      uint2 w[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r] = *reinterpret_cast<const uint2*>(wrow[r] + k);
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[m][r] += dot8_bf16_i8(a[m], w[r].x, w[r].y);
    } else {
      uint4 w[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r] = *reinterpret_cast<const uint4*>(wrow[r] + (long)k * 2);
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[m][r] += dot8_bf16(a[m], w[r]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float v = wave_sum(acc[m][r]);
      if (lane == 0) part[wave][m][r] = v;
    }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < MR * GV_P) {
    const int m = t / GV_P, q = t - m * GV_P;
    const int j = j0 + q;
    if (m < g.M && j < n_pairs) {
      float va = 0.f, vb = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        va += part[wv][m][2 * q];
        vb += part[wv][m][2 * q + 1];
      }
      int n_a, n_b;
      gv_pair_cols(g, EPI, j, n_a, n_b);
      if (BT) {  // int8 weights: per-output-channel scales
        va *= g.bscale[n_a];
        vb *= g.bscale[n_b];
      }
      epi_pair<EPI, bf16_t>(g, m, n_a, n_b, va, vb);
    }
  }
}

template <int EPI, int BT, int NORM>
hipError_t launch_gemv_n(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)((g.N / 2 + GV_P - 1) / GV_P));
  if (g.M == 1)
    hipLaunchKernelGGL((gemv_bf16_kernel<EPI, 1, BT, NORM>), grid, dim3(256), 0, s, g);
  else if (g.M == 2)
    hipLaunchKernelGGL((gemv_bf16_kernel<EPI, 2, BT, NORM>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemv_bf16_kernel<EPI, 4, BT, NORM>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int EPI, int BT>
hipError_t launch_gemv(const GemmArgs& g, hipStream_t s) {
  if (g.M > 4 || g.K % 32 != 0 || g.N % 2 != 0) return hipErrorInvalidValue;
  if (BT && !g.bscale) return hipErrorInvalidValue;
  if (g.a_f32) {  // rows normalised on load: the Q/K/V and gate/up products, whose inputs are RMSNorm rows
    if constexpr (EPI == EPI_ROPE || EPI == EPI_SWIGLU) {
      if (!g.a_gain) return hipErrorInvalidValue;
      return launch_gemv_n<EPI, BT, 1>(g, s);
    }
    return hipErrorInvalidValue;
  }
  return launch_gemv_n<EPI, BT, 0>(g, s);
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
template <int EPI, int BT>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  hipError_t e;
  switch (g.cfg) {
    case GEMM_GEMV:
      return launch_gemv<EPI, BT>(g, s);
    case GEMM_128x512:  // planned for the SwiGLU epilogue only
      if constexpr (EPI == EPI_SWIGLU) { e = launch_dma<128, 512, 2, 4, 2, EPI, BT>(g, s); break; }
      return hipErrorInvalidValue;
    case GEMM_256x256:  // fp32 outputs (residual, split-K partials) staged in row halves
      // sixteen wavefronts (four per SIMD, 64 x 64 each) hide more of the operand-load latency
      // than eight (128 x 64 each: 2-8% slower on the FFN products); the int8 weight path needs
      // the eight-wavefront register budget
      if constexpr (BT == 0) {
        // up to 4096 rows the weight tile gets a third stage (the 160 KiB of LDS hold 2
        // activation and 3 weight stages): steady 70B gate/up 2021 -> 1982 us, down 1338 ->
        // 1261 us; at 16640 rows the two-stage ring is 2% faster
        if (g.M <= 4096) e = launch_dma<256, 256, 4, 4, 2, EPI, BT, 1>(g, s);
        else e = launch_dma<256, 256, 4, 4, 2, EPI, BT, 0>(g, s);
      } else {
        e = launch_dma<256, 256, 2, 4, 2, EPI, BT>(g, s);
      }
      break;
    case GEMM_128x256: e = launch_dma<128, 256, 2, 4, 3, EPI, BT>(g, s); break;
    case GEMM_64x256: e = launch_dma<64, 256, 1, 4, 3, EPI, BT>(g, s); break;
    case GEMM_128x128: e = launch_dma<128, 128, 2, 2, 3, EPI, BT>(g, s); break;
    case GEMM_64x128: e = launch_dma<64, 128, 2, 2, 4, EPI, BT>(g, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || g.splits <= 1) return e;
  if (EPI == EPI_RESID) {
    if (g.N > 256 * kResidMaxBlocks || g.splits > 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_resid_norm_kernel, dim3(g.M), dim3(resid_norm_threads(g.N)), 0, s, g);
  } else {
    const long items = (long)g.M * (g.N / 8);
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace

// Tile of a product that does not split K.  Model: a workgroup of tile cfg takes about t(cfg)
// per 64-wide K-step whatever the shape, and the grid runs in ceil(workgroups / 256) waves; the
// tile with the fewest wave-steps wins.  t measured on MI355X (K = 1536, one wave of
// workgroups): 64x128 0.72 us, 128x128 0.83, 64x256 1.04, 128x256 1.13, 256x256 1.75, 128x512
// 2.10.  The model ranks the measured tiles of the gate/up products of the Qwen2.5-1.5B shape at
// 64..5184 rows and of the Mistral-7B shape at 640..1024 rows within 10% of the best.  128 x 512
// is built for the SwiGLU epilogue only.  Short reductions keep to bf16-output tiles for the
// residual add (256 x 256 is left out there: its fp32 tile is staged in two halves).
GemmCfg tile_by_model(int M, int N, int epi, long* workgroups) {
  struct Cand {
    GemmCfg cfg;
    int bm, bn;
    float t;
  };
  constexpr Cand cands[] = {{GEMM_64x128, 64, 128, 0.72f},   {GEMM_128x128, 128, 128, 0.83f},
                            {GEMM_64x256, 64, 256, 1.04f},   {GEMM_128x256, 128, 256, 1.13f},
                            {GEMM_256x256, 256, 256, 1.75f}, {GEMM_128x512, 128, 512, 2.10f}};
  GemmCfg best = GEMM_64x128;
  float best_cost = 3.4e38f;
  long best_wgs = (long)((M + 63) / 64) * (N / 128);
  for (const Cand& c : cands) {
    if (N % c.bn) continue;
    if (c.cfg == GEMM_128x512 && epi != EPI_SWIGLU) continue;
    if (c.cfg == GEMM_256x256 && epi == EPI_RESID) continue;
    const long wgs = (long)((M + c.bm - 1) / c.bm) * (N / c.bn);
    const float cost = (float)((wgs + 255) / 256) * c.t;
    if (cost < best_cost) {
      best_cost = cost;
      best = c.cfg;
      best_wgs = wgs;
    }
  }
  if (workgroups) *workgroups = best_wgs;
  return best;
}

// Tile configuration and split-K factor for an M x N x K product (measured on MI355X at the
// fusion step's shapes):
//   * M <= 4 rows (a decode step): the skinny product, no split;
//   * SwiGLU (gate/up, widest output): no split (the epilogue needs whole sums), the tile
//     tile_by_model ranks first (64 x 128 at 64 rows, 128 x 256 at 320, 256 x 256 at 640,
//     128 x 512 at 832, 256 x 256 from 1600 for Qwen);
//   * short reductions (K <= 2048: the Q/K/V and o-projections): the tile tile_by_model ranks
//     first (64 x 128 at 832 rows, 128 x 128 at 1600, 128 x 128 for the 512 K/V columns of all
//     5184 rows, 256 x 256 for all of Q/K/V there), no split, if it gives at least ~150
//     workgroups; else 64 x 128 tiles of 4 wavefronts with a 4-stage ring and K split up to
//     ~150 workgroups;
//   * long reductions over large M (>= 2048 rows) with N % 256 == 0: long_reduction_plan;
//   * problems with >= 200 tiles of 128 x 256: those tiles (8 wavefronts), no split;
//   * other long reductions (the FFN down-projection): up to 320 rows, 64 x 128 tiles with K
//     split so that at most 256 workgroups run (64 rows: 15 against 20 us with 64 x 256); above,
//     128 x 256 tiles, K split so that about 210 workgroups run;
//   each split keeps at least two 64-wide K-steps and its partials fit the buffer.
// Long reductions (K > 2048, N % 256 == 0): 128 x 128, 128 x 256 or 256 x 256 tiles with K
// split 1..max_split ways, the cheapest by the tile model (waves x t(cfg) per K-step x K-steps
// per split) plus what the split costs: the reduce reads the s fp32 partial planes (and, for the
// residual epilogue, the residual) and writes the output, about (s + 2) M N 4 + 2 M N bytes at
// ~4 TB/s; an unsplit residual output is followed by its own RMSNorm pass, M N 6 bytes at
// ~2.8 TB/s (the rates measured for those kernels on MI355X).  Llama-70B shape, 2714 rows: the
// down-projection (K 28672) and the o-projection (K 8192) take 256 x 256 split 2, the Q/K/V
// product 256 x 256 unsplit; at 16640 rows every product takes 256 x 256 unsplit.
struct LongCand {
  GemmCfg cfg;
  int bm, bn;
  float t;
};
constexpr LongCand kLongCands[] = {{GEMM_128x128, 128, 128, 0.83f}, {GEMM_128x256, 128, 256, 1.13f},
                                   {GEMM_256x256, 256, 256, 1.75f}};

// Modelled microseconds of a long reduction with tile c split sp ways (see long_reduction_plan).
static double long_reduction_cost(const LongCand& c, int sp, int M, int N, int K, int epi) {
  const int nk = K / 64;
  const double mn = (double)M * N;
  const long tiles = (long)((M + c.bm - 1) / c.bm) * (N / c.bn);
  double cost = (double)((tiles * sp + 255) / 256) * c.t * ((nk + sp - 1) / sp);
  if (sp > 1) cost += ((sp + 2) * mn * 4 + mn * 2) / 4.0e6;  // the reduce at 4 TB/s
  else if (epi == EPI_RESID) cost += mn * 6 / 2.8e6;        // the RMSNorm pass at 2.8 TB/s
  return cost;
}

static GemmPlan long_reduction_plan(int M, int N, int K, int epi, long partial_cap_elems, int max_split,
                                    double* cost_out) {
  const int nk = K / 64;
  GemmPlan best{GEMM_128x256, 1};
  double best_cost = 1e300;
  for (const LongCand& c : kLongCands) {
    if (N % c.bn) continue;
    for (int sp = 1; sp <= max_split; ++sp) {
      if (sp > 1 && (nk / sp < 2 || (long)sp * M * N > partial_cap_elems)) break;
      const double cost = long_reduction_cost(c, sp, M, N, K, epi);
      if (cost < best_cost) {
        best_cost = cost;
        best = GemmPlan{c.cfg, sp};
      }
    }
  }
  if (cost_out) *cost_out = best_cost;
  return best;
}

static GemmPlan gemm_plan_rule(int M, int N, int K, int epi, long partial_cap_elems) {
  GemmPlan p{GEMM_128x128, 1};
  if (M <= 4 && K % 32 == 0) {  // a few rows (decode): weight streaming on the vector ALUs
    p.cfg = GEMM_GEMV;
    return p;
  }
  if (epi == EPI_SWIGLU) {
    p.cfg = tile_by_model(M, N, epi, nullptr);
    return p;
  }
  if (K <= 2048) {
    long wgs = 0;
    p.cfg = tile_by_model(M, N, epi, &wgs);
    if (wgs >= 150) return p;
  } else if (M >= 2048 && N % 256 == 0) {
    return long_reduction_plan(M, N, K, epi, partial_cap_elems, 4, nullptr);
  }
  int bm = 128, bn = 128, target = 210;
  bool one_wave = false;  // split only as far as one wave of 256 workgroups
  if (K > 2048 && N % 256 == 0 && ((M + 127) / 128) * (N / 256) >= 200) {
    p.cfg = GEMM_128x256;
    return p;
  }
  if (K <= 2048) {
    p.cfg = GEMM_64x128;
    bm = 64;
    target = 150;
  } else if (M <= 320) {  // a long reduction over few rows: small tiles, K split up to 8 ways
    p.cfg = GEMM_64x128;
    bm = 64;
    target = 256;
    one_wave = true;
  } else if (N % 256 == 0) {
    p.cfg = GEMM_128x256;
    bn = 256;
  }
  const int tiles = ((M + bm - 1) / bm) * (N / bn);
  if (tiles < target) {
    const int nk = K / 64;
    int sp = one_wave ? target / tiles : (target + tiles - 1) / tiles;
    sp = sp > 8 ? 8 : (sp < 1 ? 1 : sp);
    while (sp > 1 && (nk / sp < 2 || (long)sp * M * N > partial_cap_elems)) --sp;
    p.splits = sp;
  }
  return p;
}

// A long reduction over more than 320 and fewer than 2048 rows keeps the rule above unless the
// cost model of long_reduction_plan (splits up to 8) predicts at least 10% less time (Llama-70B
// shape at 870 rows: Q/K/V 256 x 256 split 3, down 256 x 256 split 2; Mistral-7B at 832 and 1024
// rows: Q/K/V 128 x 256 unsplit, down 256 x 256 split 4; Yi-34B at 832: o and down 256 x 256
// split 2); the Qwen shape's products keep the rule.
GemmPlan gemm_plan(int M, int N, int K, int epi, long partial_cap_elems) {
  const GemmPlan p = gemm_plan_rule(M, N, K, epi, partial_cap_elems);
  if (epi == EPI_SWIGLU || p.cfg == GEMM_GEMV || K <= 2048 || M <= 320 || M >= 2048 || N % 256) return p;
  double model = 0.0;
  const GemmPlan q = long_reduction_plan(M, N, K, epi, partial_cap_elems, 8, &model);
  for (const LongCand& c : kLongCands)
    if (c.cfg == p.cfg && model < 0.9 * long_reduction_cost(c, p.splits, M, N, K, epi)) return q;
  return p;
}

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (g.a_f32 && g.cfg != GEMM_GEMV) return hipErrorInvalidValue;  // normalise-on-load: skinny product only
  if (g.kv_k && (g.epi != EPI_ROPE || g.kvd % 128 != 0 || g.kv_col0 % 128 != 0 || !g.kv_v || !g.sel_out ||
                 !g.local_out || !g.pos))
    return hipErrorInvalidValue;  // K/V rows scattered by the epilogue: whole heads of 128 columns
  hipError_t e;
  switch (g.epi) {
    case EPI_ROPE: e = g.b_i8 ? launch_epi<EPI_ROPE, 1>(g, s) : launch_epi<EPI_ROPE, 0>(g, s); break;
    case EPI_SWIGLU: e = g.b_i8 ? launch_epi<EPI_SWIGLU, 1>(g, s) : launch_epi<EPI_SWIGLU, 0>(g, s); break;
    case EPI_RESID: e = g.b_i8 ? launch_epi<EPI_RESID, 1>(g, s) : launch_epi<EPI_RESID, 0>(g, s); break;
    default: e = g.b_i8 ? launch_epi<EPI_STORE, 1>(g, s) : launch_epi<EPI_STORE, 0>(g, s); break;
  }
  // the RMSNorm of a residual output that was written directly (no split-K reduce)
  if (e == hipSuccess && g.epi == EPI_RESID && g.norm_out && g.splits <= 1)
    e = rmsnorm((const float*)g.out, g.ldo, g.M, g.N, g.norm_g, g.norm_eps, g.norm_out, 1, s);
  return e;
}

hipError_t gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int tiles = ((g.M + 63) / 64) * (g.N / FBN);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace cb
