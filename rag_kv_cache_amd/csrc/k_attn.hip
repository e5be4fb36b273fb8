// Sparse-query causal GQA attention (CacheBlend review: the selected tokens' queries attend,
// under the causal mask, to all available K/V; tokens that were not recomputed stay keys).
//
// Query rows are the kept rows of the layer (ascending positions qpos); keys are every fused
// K/V row 0 .. qpos[row].  bf16 path (head_dim 128):
//   workgroup = 16 x QT consecutive query rows x all G query heads of one KV head (one
//   wavefront per query head and 16-row block, so the K/V tile in LDS serves the whole GQA
//   group; QT = 2 up to 6 heads, else 1);
//   64-key tiles of K and V, row-major in a 4-stage LDS ring (loaded global -> LDS directly,
//   16-byte chunks swizzled by row);
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K as the A operand, the wave's Q rows held
//   in registers as the B operand), so every lane owns one query row's scores: lane l has
//   row (l & 15) and keys 4*(l >> 4) + r of each 16-key block;
//   online softmax in fp32 (exp2 with log2(e)/sqrt(d) folded into the scale), row max and
//   sum over the four lanes of a row by two lane swaps (permlane16/32), the reference maximum
//   moved (and O rescaled) only when a score exceeds it by more than 2^8 in probability;
//   O^T += V^T P^T: P (rounded to bf16) is already in B-operand layout, V^T fragments come
//   from LDS transpose reads of the row-major V tile;
//   split-KV: grid.y splits the key range so short query sets still fill the chip; a split
//   writes its output divided by its own softmax sum, in fp16, and its (max, sum) in fp32;
//   attn_combine_kernel merges the splits of each row.
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

typedef _Float16 half_t;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two floats as packed fp16 (round to nearest even), low half = lo.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(half_t)lo, (half_t)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float4 unpack_f16x4(const u32x2_t p) {
  // through scalar temporaries: a bit cast of a vector element subscript (p[1]) reads element 0
  const uint32_t lo = p.x, hi = p.y;
  const f16x2_t a = __builtin_bit_cast(f16x2_t, lo), b = __builtin_bit_cast(f16x2_t, hi);
  return make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
}

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one query row, with gfx950's
// lane-swap instructions (VALU, no LDS crossbar); every lane gets the same value.
__device__ __forceinline__ float max4_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {  // s_waitcnt vmcnt(N), other counters not waited
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Swizzles of the K and V tile rows (256 bytes, sixteen 16-byte chunks): a row's chunk c sits in
// slot c ^ swz(row).  K (read with ds_read_b128, 16 rows of one chunk per instruction) uses
// row & 15; V (read with the ds_read_b64_tr_b16 transpose, 16 rows x 32 bytes per instruction)
// uses 2 (row & 7) + (row >> 3 & 1), which puts the chunk pairs of 8 consecutive rows in 8
// distinct pairs of slots.  Measured with SQ_LDS_BANK_CONFLICT: the V reads with row & 15 stalled
// 1.8 M cycles per steady-layer launch, with this swizzle none; the K reads show none with
// row & 15 (the other swizzles tried for K conflicted).
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

constexpr int ATT_NS = 4;                     // LDS stages (K + V tile each)
constexpr float ATT_LAZY = 8.f;               // probabilities against a stale maximum stay <= 2^8
constexpr int ATT_STAGE_B = 2 * 64 * 256;     // 64 keys x 256 B (one head) for K, then V

template <int G, int RB, int QT>
__global__ __launch_bounds__(64 * G * QT) void attn_bf16_kernel(AttnArgs a) {
  constexpr int DH = 128, BKV = 64, BQ = 16 * RB * QT, NW = G * QT;
  constexpr int ROWB = DH * 2;                       // 256 bytes per K/V row
  constexpr int TILE_B = BKV * ROWB;
  constexpr int NINS = 2 * TILE_B / 1024;            // 1 KB wave instructions per K+V tile
  constexpr int INS_HI = (NINS + NW - 1) / NW, INS_LO = NINS / NW, N_HI = NINS % NW;
  extern __shared__ __align__(16) unsigned char smem[];

  // workgroups go out heaviest first (the last key range, then the last row blocks, which have
  // the most keys under the causal mask), so that the short ones fill the tail (~1.5% on the
  // 70B steady layer); the results do not depend on the order
  const int qt = (int)(gridDim.x / a.hkv) - 1 - (int)(blockIdx.x / a.hkv);
  const int g = blockIdx.x - (blockIdx.x / a.hkv) * a.hkv;
  const int split = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int row0 = qt * BQ;
  const int last = min(row0 + BQ, a.n_q) - 1;
  const int maxpos = a.qpos[last];
  const int kbeg = split * a.split_len;
  if (kbeg > maxpos) return;
  const int kend = min(min(kbeg + a.split_len, maxpos + 1), a.n_tok);
  const int minpos = a.qpos[row0];
  const int nt = (kend - kbeg + BKV - 1) / BKV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = g * G + wave % G;          // query head of this wave
  const int wrow0 = row0 + (wave / G) * 16 * RB;  // first query row of this wave
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q);
  const long kv_row_b = (long)a.hkv * ROWB;
  const float c = a.scale_log2;

  // This wave's load instructions: ids wave, wave + NW, ...; id < 16 loads K rows 4*id.., else V.
  // Lane l writes 16 bytes at slot l of the 1 KB block: row 4*(id%16) + l/16, slot l%16 holding
  // the row's 16-byte chunk (l%16) ^ swz(row) (swz_k for K, swz_v for V).
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // the same value, in a scalar register: the
                                                        // buffer descriptor chosen from it is uniform
  const int my_ins = wv < N_HI ? INS_HI : INS_LO;
  // Loads go through buffer descriptors over the n_tok rows of K and of V: a lane's byte offset
  // within the tile is fixed, the tile's offset is scalar, so a load costs no vector ALU work.
  // Keys past the split's range are loaded too (fused rows, or zeros past row n_tok from the
  // descriptor's bound) and get probability 0 from the mask.
  int ld_lds[INS_HI];
  uint32_t ld_voff[INS_HI];
  bool ld_k[INS_HI];
#pragma unroll
  for (int i = 0; i < INS_HI; ++i) {
    const int id = wv + NW * i;
    const int blk = id & 15;
    const int row = 4 * blk + (lane >> 4);
    const int chunk = (lane & 15) ^ (id < 16 ? swz_k(row) : swz_v(row));
    ld_voff[i] = (uint32_t)(row * kv_row_b + g * ROWB + chunk * 16);
    ld_k[i] = id < 16;
    ld_lds[i] = (id < 16 ? 0 : TILE_B) + blk * 1024;
  }
  const int kv_bytes = (int)((long)a.n_tok * kv_row_b);
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int kt = kbeg + t * BKV;
    unsigned char* st = smem + (t % ATT_NS) * ATT_STAGE_B;
    const int soff = (int)(kt * kv_row_b);
#pragma unroll
    for (int i = 0; i < INS_HI; ++i)
      if (i < my_ins) buffer_load_lds16(ld_k[i] ? a.k : a.v, kv_bytes, st + ld_lds[i], ld_voff[i], soff);
  };
  // wait until tile t+1 has landed, with `more` = whether tile t+2 was issued after it (waves
  // that issued INS_HI loads per tile wait for one load of tile t+2 too: over-waiting is safe)
  auto wait_next = [&](bool more) __attribute__((always_inline)) {
    if (more) wait_vmcnt<INS_LO>();
    else wait_vmcnt<0>();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  int mypos[RB];
  bf16x8_t qf[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wrow0 + rb * 16 + l16;
    const bool ok = r < a.n_q;
    mypos[rb] = ok ? a.qpos[r] : -1;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qf[rb][ds] = ok ? *reinterpret_cast<const bf16x8_t*>(Q + (long)r * a.ldq + h * DH + ds * 32 + lg * 8)
                      : bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
  float m_i[RB], l_i[RB];
  f32x4_t o[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_i[rb] = NEG_INF;
    l_i[rb] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[rb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // S^T = K Q^T for the tile in stage st: s[rb][kb][r] = score of row rb*16+l16, key 16kb+4lg+r.
  // Dimension steps outside, key blocks inside: four independent accumulation chains.
  auto qk = [&](int t, f32x4_t (&s)[RB][4]) __attribute__((always_inline)) {
    const unsigned char* kb_ = smem + (t % ATT_NS) * ATT_STAGE_B;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const int chunk = ds * 4 + lg;
      bf16x8_t ka[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = kb * 16 + l16;
        ka[kb] = *reinterpret_cast<const bf16x8_t*>(kb_ + row * ROWB + ((chunk ^ swz_k(row)) << 4));
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qf[rb][ds], s[rb][kb], 0, 0, 0);
    }
  };
  // online softmax of tile t's scores, then O += V P for that tile
  auto softmax_pv = [&](int t, f32x4_t (&s)[RB][4]) __attribute__((always_inline)) {
    const int kt = kbeg + t * BKV;
    const bool edge = (kt + BKV > kend) || (kt + BKV - 1 > minpos);
    bf16x8_t pf[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (edge) {
        const int thr = min(mypos[rb], kend - 1) - kt - 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[rb][kb][r] = (kb * 16 + r <= thr) ? s[rb][kb][r] : NEG_INF;
      }
      // this lane's 16 scores: a chain of 3-input maxima (v_max3_f32, 8 instructions)
      float mx = fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), s[rb][0][2]);
#pragma unroll
      for (int j = 3; j < 15; j += 2)
        mx = fmaxf(fmaxf(mx, s[rb][j >> 2][j & 3]), s[rb][(j + 1) >> 2][(j + 1) & 3]);
      mx = fmaxf(mx, s[rb][3][3]);
      mx = max4_rows(mx);
      const float m_new = fmaxf(m_i[rb], mx);
      // Lazy rescaling: the reference maximum m_i moves only when a row of the wavefront sees a
      // scaled score more than ATT_LAZY (log2 units) above it; until then the probabilities are
      // taken against the older reference (at most 2^ATT_LAZY), which leaves O / l unchanged and
      // skips the rescale of O.  A row's first valid keys always move it (from -inf).
      if (__ballot((m_new - m_i[rb]) * c > ATT_LAZY)) {
        const float alpha = (m_new == m_i[rb]) ? 1.f : __builtin_amdgcn_exp2f((m_i[rb] - m_new) * c);
        l_i[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[rb][d] *= alpha;
        m_i[rb] = m_new;
      }
      const float mc = (m_i[rb] == NEG_INF) ? 0.f : m_i[rb] * c;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[rb][kb][r], c, -mc));
          s[rb][kb][r] = p;
          rs += p;
        }
      l_i[rb] += rs;  // this lane's share of the row sum (reduced at the end)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4_t w = {pack_bf16x2(s[rb][2 * ks][0], s[rb][2 * ks][1]), pack_bf16x2(s[rb][2 * ks][2], s[rb][2 * ks][3]),
                           pack_bf16x2(s[rb][2 * ks + 1][0], s[rb][2 * ks + 1][1]),
                           pack_bf16x2(s[rb][2 * ks + 1][2], s[rb][2 * ks + 1][3])};
        pf[rb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // V^T fragments by transpose reads: lane (group lg, j = l16) reads 8 bytes of key row
    // 32ks + 4lg + j/4 (+16), dims 16d + 4(j%4); it receives V[4 keys][dim 16d + j].
    const unsigned char* vb_ = smem + (t % ATT_NS) * ATT_STAGE_B + TILE_B;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int row = ks * 32 + 4 * lg + (l16 >> 2);
        const int chunk = 2 * d + ((l16 & 3) >> 1);
        const int byte = (l16 & 1) * 8;
        const u32x2_t lo = lds_read_tr16(reinterpret_cast<const bf16_t*>(vb_ + row * ROWB + ((chunk ^ swz_v(row)) << 4) + byte));
        const int row2 = row + 16;
        const u32x2_t hi = lds_read_tr16(reinterpret_cast<const bf16_t*>(vb_ + row2 * ROWB + ((chunk ^ swz_v(row2)) << 4) + byte));
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[rb][ks], o[rb][d], 0, 0, 0);
      }
  };

  // Prologue: tiles 0..2 in flight, wait for tile 0, scores of tile 0.
  issue(0);
  if (nt > 1) issue(1);
  if (nt > 2) issue(2);
  if (nt > 2) wait_vmcnt<2 * INS_LO>();
  else if (nt > 1) wait_vmcnt<INS_LO>();
  else wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  f32x4_t sa[RB][4], sb[RB][4];
  qk(0, sa);
  // Iteration t: tile t+1 landed -> barrier; refill the stage of tile t-1 with tile t+3; scores of
  // tile t+1 (MFMA) next to the softmax of tile t (VALU); then O += V_t P_t.
  for (int t = 0; t < nt; t += 2) {
    if (t + 1 < nt) {
      wait_next(t + 2 < nt);
      if (t + 3 < nt) issue(t + 3);
      qk(t + 1, sb);
    }
    softmax_pv(t, sa);
    if (t + 1 >= nt) break;
    if (t + 2 < nt) {
      wait_next(t + 3 < nt);
      if (t + 4 < nt) issue(t + 4);
      qk(t + 2, sa);
    }
    softmax_pv(t + 1, sb);
  }

  // o[rb][d][r] = O[row rb*16 + l16][d*16 + 4*lg + r]; the row sum is spread over 4 lanes
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l_i[rb] = sum4_rows(l_i[rb]);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int my_row = wrow0 + rb * 16 + l16;
    if (my_row >= a.n_q) continue;
    if (a.splits == 1) {
      const float inv = l_i[rb] > 0.f ? 1.f / l_i[rb] : 0.f;
      bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + (long)my_row * a.ldo + h * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<u32x2_t*>(out + d * 16) =
            u32x2_t{pack_bf16x2(o[rb][d][0] * inv, o[rb][d][1] * inv), pack_bf16x2(o[rb][d][2] * inv, o[rb][d][3] * inv)};
    } else {  // the split's O normalized by its own sum, as fp16 (|O| <= max |V|), and (max, sum)
      const float inv = l_i[rb] > 0.f ? 1.f / l_i[rb] : 0.f;
      const long idx = ((long)split * a.n_q + my_row) * a.hq + h;
      half_t* po = reinterpret_cast<half_t*>(a.part_o) + idx * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<u32x2_t*>(po + d * 16) =
            u32x2_t{pack_f16x2(o[rb][d][0] * inv, o[rb][d][1] * inv), pack_f16x2(o[rb][d][2] * inv, o[rb][d][3] * inv)};
      if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(m_i[rb] * c, l_i[rb]);
    }
  }
}

// Merge split-KV partials: out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  Only splits
// whose first key is <= the row's position hold keys of that row.  One thread per
// (row, head, 4 dims); the (m, l) and O partials are summed in split order.  NB = 1: up to 8
// splits, every load issued at once; NB = 0: any number of splits, 8 at a time, in two passes
// (maxima, then the weighted sum).  Separate instantiations, so that the few-split case keeps
// its small register footprint (issuing 32 splits' loads at once measured no faster than the
// two passes).
template <typename TO, int NB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int NSB = 8;  // splits per batch of loads
  const int d4n = a.dh / 4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.n_q * a.hq * d4n;
  if (idx >= total) return;
  const int row = (int)(idx / ((long)a.hq * d4n));
  const int rem = (int)(idx - (long)row * a.hq * d4n);
  const int h = rem / d4n, d0 = (rem - h * d4n) * 4;
  const int ns = min(a.qpos[row] / a.split_len + 1, a.splits);
  const half_t* part = reinterpret_cast<const half_t*>(a.part_o);
  float M = NEG_INF, L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto load = [&](int s0, float2 (&ml)[NSB], float4 (&v)[NSB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NSB; ++j) {
      if (s0 + j < ns) {
        const long pi = ((long)(s0 + j) * a.n_q + row) * a.hq + h;
        ml[j] = *reinterpret_cast<const float2*>(a.part_ml + pi * 2);
        const u32x2_t hv = *reinterpret_cast<const u32x2_t*>(part + pi * a.dh + d0);
        v[j] = unpack_f16x4(hv);
      } else {
        ml[j] = make_float2(NEG_INF, 0.f);
      }
    }
  };
  // O_s holds the split's sum-normalized output: the weight of split s is l_s 2^(m_s - M)
  auto add = [&](const float2 (&ml)[NSB], const float4 (&v)[NSB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NSB; ++j) {
      if (ml[j].x == NEG_INF) continue;
      const float w = ml[j].y * exp2f(ml[j].x - M);
      L += w;
      acc[0] += v[j].x * w; acc[1] += v[j].y * w; acc[2] += v[j].z * w; acc[3] += v[j].w * w;
    }
  };
  if constexpr (NB > 0) {  // NB batches, every load issued before any is used
    float2 ml[NB][NSB];
    float4 v[NB][NSB];
#pragma unroll
    for (int b = 0; b < NB; ++b) load(b * NSB, ml[b], v[b]);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < NSB; ++j) M = fmaxf(M, ml[b][j].x);
#pragma unroll
    for (int b = 0; b < NB; ++b) add(ml[b], v[b]);
  } else {
    for (int s0 = 0; s0 < ns; s0 += NSB) {  // the splits' maxima, a batch of loads at a time
      float mv[NSB];
#pragma unroll
      for (int j = 0; j < NSB; ++j)
        mv[j] = s0 + j < ns ? a.part_ml[(((long)(s0 + j) * a.n_q + row) * a.hq + h) * 2] : NEG_INF;
#pragma unroll
      for (int j = 0; j < NSB; ++j) M = fmaxf(M, mv[j]);
    }
    for (int s0 = 0; s0 < ns; s0 += NSB) {
      float2 ml[NSB];
      float4 v[NSB];
      load(s0, ml, v);
      add(ml, v);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  TO* out = reinterpret_cast<TO*>(a.out) + (long)row * a.ldo + h * a.dh + d0;
#pragma unroll
  for (int i = 0; i < 4; ++i) Elem<TO>::st(out + i, acc[i] * inv);
}

// ---------------------------------------------------------------- decode (few query rows)
// A decode step has 1..4 query rows: 16-row MFMA tiles would be almost empty, so the few rows
// run on the vector ALUs with the key range split finely.  One workgroup per (KV head g, key
// range sp), 4 wavefronts; 16 lanes hold one key row (8 of its 128 dims each), so a wavefront
// takes 4 keys per step and the workgroup 16.  Every lane keeps, for each of the MR rows x G
// query heads of the group, the online-softmax state (max, sum, 8 dims of O) of the keys its
// 16-lane row sees; the states are merged across the 4 rows of a wavefront with lane swaps and
// across wavefronts in LDS, and written as the split's partial (O, max, sum) for the combine.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes, every lane getting the row's sum.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f<0x141>(v);  // row_half_mirror: lane i of 8 reads 7 - i, i.e. the other quad
  v += dpp_f<0x140>(v);  // row_mirror: lane i of 16 reads 15 - i, i.e. the other 8 lanes
  return v;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int G, int MR>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a) {
  constexpr int DH = 128, RH = MR * G;
  __shared__ float s_o[4][RH][DH];
  __shared__ float s_m[4][RH], s_l[4][RH];
  const int g = blockIdx.x, sp = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane >> 4, dl = (lane & 15) * 8;
  const int k0 = sp * a.split_len;
  const int kend0 = min(k0 + a.split_len, a.n_tok);
  const long rs = (long)a.hkv * DH;  // elements per fused row
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + g * DH + dl;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + g * DH + dl;
  // Every load of the first DU steps is issued before any is used (K/V rows, Q, positions), so
  // the workgroup waits for memory once; rows' causal bounds are applied afterwards.
  // The 16 lanes of a row share kb, so a row is wholly active or inactive (DPP stays in rows).
  constexpr int DU = 8;
  int kb0 = k0 + wave * 4 + kl;
  uint4 kr[DU], vr[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    const int kb = kb0 + 16 * u;
    if (kb < kend0) {
      kr[u] = *reinterpret_cast<const uint4*>(K + kb * rs);
      vr[u] = *reinterpret_cast<const uint4*>(V + kb * rs);
    }
  }
  uint4 qraw[MR][G];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (r < a.n_q)
        qraw[r][h] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.q) + (long)r * a.ldq +
                                                     (g * G + h) * DH + dl);
  int qp[MR];
  int qmax = -1;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    qp[r] = r < a.n_q ? a.qpos[r] : -1;
    qmax = max(qmax, qp[r]);
  }
  const int kend = min(kend0, qmax + 1);
  if (k0 >= kend) return;  // no row attends to this key range (uniform over the workgroup)

  float q[MR][G][8];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (r < a.n_q) {
        unpack_bf16x8(qraw[r][h], q[r][h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[r][h][e] *= a.scale_log2;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[r][h][e] = 0.f;
      }
    }
  float m[MR][G], l[MR][G], o[MR][G][8];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[r][h] = NEG_INF;
      l[r][h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][h][e] = 0.f;
    }
  for (;;) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int kb = kb0 + 16 * u;
      if (kb >= kend) break;
      float kf[8], vf[8];
      unpack_bf16x8(kr[u], kf);
      unpack_bf16x8(vr[u], vf);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const bool live = kb <= qp[r];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sc = fmaf(q[r][h][e], kf[e], sc);
          sc = sum16(sc);
          if (live) {
            const float mn = fmaxf(m[r][h], sc);
            const float al = __builtin_amdgcn_exp2f(m[r][h] - mn);  // exp2(-inf) = 0
            const float p = __builtin_amdgcn_exp2f(sc - mn);
            l[r][h] = l[r][h] * al + p;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[r][h][e] = fmaf(p, vf[e], o[r][h][e] * al);
            m[r][h] = mn;
          }
        }
      }
    }
    kb0 += 16 * DU;
    if (kb0 >= kend) break;
    // key ranges longer than 16 DU keys: the next DU steps
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int kb = kb0 + 16 * u;
      if (kb < kend) {
        kr[u] = *reinterpret_cast<const uint4*>(K + kb * rs);
        vr[u] = *reinterpret_cast<const uint4*>(V + kb * rs);
      }
    }
  }
  // merge the 4 key rows of the wavefront (lanes l, l^16, l^32, l^48 hold the same dims)
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float M = max4_rows(m[r][h]);
      const float w = m[r][h] == NEG_INF ? 0.f : exp2f(m[r][h] - M);
      const float L = sum4_rows(l[r][h] * w);
      float od[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) od[e] = sum4_rows(o[r][h][e] * w);
      if (kl == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[wave][r * G + h][dl + e] = od[e];
        if (lane == 0) {
          s_m[wave][r * G + h] = M;
          s_l[wave][r * G + h] = L;
        }
      }
    }
  __syncthreads();
  // merge the wavefronts and write the split's partial of every row that reads this split
  for (int i = threadIdx.x; i < RH * DH; i += 256) {
    const int rh = i / DH, d = i - rh * DH;
    const int r = rh / G, h = rh - r * G;
    if (r >= a.n_q || qp[r] < k0) continue;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][rh]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = s_m[w][rh] == NEG_INF ? 0.f : exp2f(s_m[w][rh] - M);
      O = fmaf(wt, s_o[w][rh][d], O);
      L = fmaf(wt, s_l[w][rh], L);
    }
    const long pi = ((long)sp * a.n_q + r) * a.hq + g * G + h;
    a.part_o[pi * DH + d] = O;
    if (d == 0) {
      a.part_ml[pi * 2] = M;
      a.part_ml[pi * 2 + 1] = L;
    }
  }
}

// Combine of the decode partials: one workgroup of DH threads per (row, query head); the
// splits' (max, sum) go through LDS, then each thread sums its dim over the row's splits with
// every load in flight at once (at most kDecodeMaxSplits).
constexpr int kDecodeMaxSplits = 64;
template <typename TO>
__global__ __launch_bounds__(128) void attn_combine_few_kernel(AttnArgs a) {
  __shared__ float s_w[kDecodeMaxSplits];
  __shared__ float s_inv;
  const int row = blockIdx.x / a.hq, h = blockIdx.x - row * a.hq;
  const int t = threadIdx.x;
  const int nsp = min(a.splits, kDecodeMaxSplits);
  // every load at once (positions, the splits' (max, sum), this thread's dim of every split's O);
  // splits past the row's last one are not read further (their buffers may hold anything)
  float v[kDecodeMaxSplits];
#pragma unroll
  for (int sidx = 0; sidx < kDecodeMaxSplits; ++sidx)
    if (sidx < nsp) v[sidx] = a.part_o[(((long)sidx * a.n_q + row) * a.hq + h) * a.dh + t];
  float2 mlv = make_float2(NEG_INF, 0.f);
  if (t < nsp) mlv = *reinterpret_cast<const float2*>(a.part_ml + (((long)t * a.n_q + row) * a.hq + h) * 2);
  const int ns = min(a.qpos[row] / a.split_len + 1, nsp);
  if (t < 64) {  // wavefront 0 holds every split's (max, sum)
    const float mv = t < ns ? mlv.x : NEG_INF, lv = t < ns ? mlv.y : 0.f;
    float M = mv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = mv == NEG_INF ? 0.f : exp2f(mv - M);
    const float L = wave_sum(lv * w);
    s_w[t] = w;
    if (t == 0) s_inv = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int sidx = 0; sidx < kDecodeMaxSplits; ++sidx)
    if (sidx < ns) acc = fmaf(s_w[sidx], v[sidx], acc);
  Elem<TO>::st(reinterpret_cast<TO*>(a.out) + (long)row * a.ldo + h * a.dh + t, acc * s_inv);
}

template <int G, int MR>
hipError_t launch_decode(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_kernel<G, MR>), dim3(a.hkv, a.splits), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_few_kernel<bf16_t>, dim3(a.n_q * a.hq), dim3(128), 0, s, a);
  return hipGetLastError();
}

// The decode kernel for n_q query rows of group G when its registers allow (MR x G <= 8, MR
// the row count rounded up to 1, 2 or 4); hipErrorNotSupported otherwise.
template <int G>
hipError_t launch_decode_g(const AttnArgs& a, hipStream_t s) {
  if (a.n_q == 1 && G <= 8) return launch_decode<G, 1>(a, s);
  if constexpr (2 * G <= 8) {
    if (a.n_q == 2) return launch_decode<G, 2>(a, s);
  }
  if constexpr (4 * G <= 8) {
    if (a.n_q <= 4) return launch_decode<G, 4>(a, s);
  }
  return hipErrorNotSupported;
}

// fp32 path (correctness configurations): one thread per (query row, query head), online
// softmax over keys 0 .. qpos[row], head_dim DH in registers.
template <int DH>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_q * a.hq) return;
  const int row = idx / a.hq, h = idx - row * a.hq;
  const int g = h / (a.hq / a.hkv);
  const int kend = min(a.qpos[row] + 1, a.n_tok);
  const float* q = reinterpret_cast<const float*>(a.q) + (long)row * a.ldq + h * DH;
  const float* K = reinterpret_cast<const float*>(a.k) + (long)g * DH;
  const float* V = reinterpret_cast<const float*>(a.v) + (long)g * DH;
  const long kv_row = (long)a.hkv * DH;
  float qr[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) { qr[d] = q[d]; acc[d] = 0.f; }
  float m = NEG_INF, l = 0.f;
  for (int key = 0; key < kend; ++key) {
    const float* kr = K + key * kv_row;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) s = fmaf(qr[d], kr[d], s);
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
    const float* vr = V + key * kv_row;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* out = reinterpret_cast<float*>(a.out) + (long)row * a.ldo + h * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) out[d] = acc[d] * inv;
}

template <int G, int RB, int QT>
hipError_t launch_gr(const AttnArgs& a, hipStream_t s) {
  constexpr int lds = ATT_NS * ATT_STAGE_B;
  if ((long)a.n_tok * a.hkv * 128 * 2 >= (1L << 31)) return hipErrorInvalidValue;  // 32-bit buffer offsets
  // once per process (a function-local static is initialised once, also under concurrent calls)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)attn_bf16_kernel<G, RB, QT>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  constexpr int BQ = 16 * RB * QT;
  dim3 grid(((a.n_q + BQ - 1) / BQ) * a.hkv, a.splits);
  hipLaunchKernelGGL((attn_bf16_kernel<G, RB, QT>), grid, dim3(64 * G * QT), lds, s, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
  if constexpr (G >= 7) {
    // one wavefront per head with two 16-row blocks: each K or V fragment read from LDS feeds
    // two MFMAs (the tile's LDS reads per MFMA halve); G wavefronts of ~200 registers
    return launch_gr<G, 2, 1>(a, s);
  } else {
    constexpr int QT = G <= 6 ? 2 : 1;  // 12 wavefronts at most: more would cap registers below need
    return launch_gr<G, 1, QT>(a, s);
  }
}

}  // namespace

int attn_rows_per_wg(int group) { return group <= 6 ? 32 : 32; }

// Whether the vector-ALU decode kernel takes n_q query rows of a GQA group of `group` heads.
bool attn_decode_fits(int n_q, int group) {
  if (n_q < 1 || n_q > 4) return false;
  const int mr = n_q == 1 ? 1 : (n_q == 2 ? 2 : 4);
  return mr * group <= 8;
}

hipError_t attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  hipError_t e;
  if (a.dh == 128 && attn_decode_fits(a.n_q, a.hq / a.hkv) && a.splits <= kDecodeMaxSplits) {
    switch (a.hq / a.hkv) {
      case 1: return launch_decode_g<1>(a, s);
      case 2: return launch_decode_g<2>(a, s);
      case 4: return launch_decode_g<4>(a, s);
      case 6: return launch_decode_g<6>(a, s);
      case 7: return launch_decode_g<7>(a, s);
      case 8: return launch_decode_g<8>(a, s);
      default: break;
    }
  }
  switch (a.hq / a.hkv) {
    case 1: e = launch_g<1>(a, s); break;
    case 2: e = launch_g<2>(a, s); break;
    case 4: e = launch_g<4>(a, s); break;
    case 6: e = launch_g<6>(a, s); break;
    case 7: e = launch_g<7>(a, s); break;
    case 8: e = launch_g<8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.splits <= 1) return e;
  const long total = (long)a.n_q * a.hq * (a.dh / 4);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (a.splits <= 8)
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  const int n = a.n_q * a.hq;
  dim3 grid((n + 127) / 128);
  if (a.dh == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(128), 0, s, a);
  else if (a.dh == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(128), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cb
