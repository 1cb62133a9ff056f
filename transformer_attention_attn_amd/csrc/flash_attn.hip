// Tiled online-softmax ("flash") attention forward for gfx950.
//
// One kernel template serves two callers:
//   * the non-causal encoder (q/k/v [B,H,S,D] bf16 or fp32, optional additive
//     key mask, fused residual-add epilogue);
//   * the history-only GQA prefill over a paged FP8 (e4m3fn) KV cache, whose
//     G query heads per KV head are packed into the M dimension (rows r of a KV
//     head are (head g, token t) with r = g*Lq + t).
//
// Prefill Context-Parallel Attention POC for Trainium2, "Layout": Q heads that
// share a KV head are packed together, online max/sum stay fp32 while the
// probabilities are bf16 with fp32 accumulation, and keys past
// actual_history_len receive an additive -inf bias.  Here the bias is
// derived inside the kernel from the length and cache blocks wholly past it
// are never read.
//
// Per workgroup: BM = 32*NT*RG query rows, RG row-group waves times NSPLIT
// key-split waves.  Split s handles key tiles s, s+NSPLIT, ...; the splits
// are merged through LDS at the end (log-sum-exp merge).  Each wave owns
// 32*NT rows; its Q fragments stay in registers for the whole loop.
//
// Per key tile (BN keys), per wave:
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, query rows on N), so
//   every lane owns one query row (lane % 32) and 16 keys per 32-key block;
//   row max: in-lane max + one v_permlane32_swap with the partner lane;
//   P = exp2(S*c - m) with the scale folded into one FMA (c > 0, log2 units),
//   packed to bf16 straight into the B operand of O^T += V^T P^T (d on M,
//   rows on N): P never leaves registers; the row sum is taken on the packed
//   bf16 P with v_dot2_f32_bf16, so it normalises exactly the values that were
//   multiplied into V.
// K tiles sit in LDS as [key][d] (16-byte chunks XOR-swizzled by key); V tiles
// as [key][d] too, rows padded by 64 bytes, and the A operand of the PV MFMA
// (d on M, keys on K) is read transposed with ds_read_b64_tr_b16: the padding
// puts the four keys one read touches in four different 64-byte bank groups,
// so both the plain 16-byte V writes and the transposing reads are
// conflict-free.  Global loads for the next PF tiles stay in flight in
// registers (uniform 64-bit base + 32-bit per-thread offset) while a tile is
// computed from one LDS stage and the next is written to the other.
#include "device_common.h"
#include "launch.h"

namespace mi355 {

constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

template <int D_, int BN_, int NT_, int RG_, int NSPLIT_, int GRP_, int PF_, int OCC_ = 2>
struct Geo {
  static constexpr int D = D_, BN = BN_, NT = NT_, RG = RG_, NSPLIT = NSPLIT_;
  static constexpr int GRP = GRP_;  // LDS fragments read per pipelined group
  static constexpr int PF = PF_;    // key tiles in flight in registers (global-load prefetch depth)
  static constexpr int WAVES = RG * NSPLIT, THREADS = 64 * WAVES;
  static constexpr int WPE = OCC_;  // waves per SIMD the kernel is compiled for (register budget 512 / WPE)
  static constexpr int BM = 32 * NT * RG;
  static constexpr int KT = BN * D * 2;  // bytes of one bf16 K tile
  static constexpr int VROW = D * 2 + 64;  // bytes per key row of a V tile (64-byte pad: an odd multiple of 64 mod 256)
  static constexpr int VT = BN * VROW;   // bytes of one bf16 V tile
  static constexpr int SPLIT_BYTES = KT + VT;
  static constexpr int STAGE = NSPLIT * SPLIT_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int KB = BN / 32;  // 32-key blocks per tile
  static constexpr int SD = D / 16;   // k-steps of the QK^T contraction
  static constexpr int MT = D / 32;   // d tiles of O^T
  static_assert(D % 64 == 0 && BN % 32 == 0, "tile shape");
  static_assert(LDS <= 160 * 1024, "LDS budget (gfx950: 160 KiB per workgroup)");
  static_assert((VROW / 64) % 2 == 1 && VROW % 256 != 0, "V row pad");

  // byte offset of 16-byte chunk c of key row `key` in a K tile
  static __device__ __forceinline__ int k_off(int key, int c) { return key * (D * 2) + ((c ^ (key & 7)) << 4); }
};

// ------------------------------------------------------------------ sources

// Encoder K/V: [B,H,S_kv,D] strided, bf16 or fp32 (fp32 rounded to bf16 here).
// Unit u of an iteration belongs to split u / KU; its key row is fixed per
// thread, so the address is base(iteration) + a 32-bit per-thread offset.
template <class G, bool F32>
struct EncSrc {
  const char *kb, *vb;       // this (b,h)'s K and V base
  int64_t kstep, vstep;      // bytes between consecutive iterations (NSPLIT*BN keys)
  int64_t ks, vs;            // element stride between keys
  int n_keys;
  const float *mask;         // nullable: V rows of -inf-masked keys are not loaded (zeros)
  static constexpr int ES = F32 ? 4 : 2;
  static constexpr int KU = G::BN * (G::D / 8);  // K (and V) units of 8 elements of one key per tile
  static constexpr int UK = G::NSPLIT * KU / G::THREADS;
  static_assert(UK * G::THREADS == G::NSPLIT * KU, "units");
  static constexpr int W = F32 ? 2 : 1;  // 16-byte loads per 8 elements
  struct Stage {
    u32x4_t k[UK][W];
    u32x4_t v[UK][W];
  };

  __device__ __forceinline__ int64_t tile_base(int) const { return 0; }

  __device__ __forceinline__ void load(Stage &st, int it, int64_t, int tid) const {
    asm volatile("" : "+v"(tid));  // per-thread offsets are cheap 32-bit math: recompute, don't keep live
    const char *kbase = kb + it * kstep;
    const char *vbase = vb + it * vstep;
    const int key_it = it * G::NSPLIT * G::BN;
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const int u = tid + j * G::THREADS;
      const int sp = u / KU, w = u % KU;
      const int t = sp * G::BN + w / (G::D / 8), c = w % (G::D / 8);
      const uint32_t off = (uint32_t)(t * ks + 8 * c) * ES;
#pragma unroll
      for (int x = 0; x < W; ++x)
        st.k[j][x] = key_it + t < n_keys ? ldg<u32x4_t>(kbase + off + 16 * x) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const int u = tid + j * G::THREADS;
      const int sp = u / KU, w = u % KU;
      const int t = sp * G::BN + w / (G::D / 8), c = w % (G::D / 8);
      const uint32_t off = (uint32_t)(t * vs + 8 * c) * ES;
      const int key = key_it + t;
      const bool live = key < n_keys && (mask == nullptr || mask[key] != -INFINITY);
#pragma unroll
      for (int x = 0; x < W; ++x) st.v[j][x] = live ? ldg<u32x4_t>(vbase + off + 16 * x) : u32x4_t{0, 0, 0, 0};
    }
  }

  // 8 elements of a raw unit -> 4 packed bf16 pairs (element order kept)
  static __device__ __forceinline__ u32x4_t to_bf16(const u32x4_t (&x)[W]) {
    if constexpr (F32) {
      return u32x4_t{pack_bf16(__uint_as_float(x[0][0]), __uint_as_float(x[0][1])),
                     pack_bf16(__uint_as_float(x[0][2]), __uint_as_float(x[0][3])),
                     pack_bf16(__uint_as_float(x[1][0]), __uint_as_float(x[1][1])),
                     pack_bf16(__uint_as_float(x[1][2]), __uint_as_float(x[1][3]))};
    } else {
      return x[0];
    }
  }

  __device__ __forceinline__ void store(const Stage &st, char *stage, int tid) const {
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const int u = tid + j * G::THREADS;
      const int sp = u / KU, w = u % KU;
      const int t = w / (G::D / 8), c = w % (G::D / 8);
      char *split = stage + sp * G::SPLIT_BYTES;
      *reinterpret_cast<u32x4_t *>(split + G::k_off(t, c)) = to_bf16(st.k[j]);
      *reinterpret_cast<u32x4_t *>(split + G::KT + t * G::VROW + 16 * c) = to_bf16(st.v[j]);
    }
  }
};

// Paged FP8 K/V: cache [num_blocks, Hkv, bs, D] e4m3fn; a K or V unit is 16
// fp8 of one key.  Converted to bf16 exactly on store.
template <class G>
struct PagedSrc {
  const uint8_t *kc, *vc;
  const __attribute__((address_space(4))) int32_t *bt;  // constant address space: scalar loads
  int64_t head_off;    // kvh * bs * D
  int64_t blk_stride;  // Hkv * bs * D
  int bs, n_keys;
  static constexpr int KU = G::BN * (G::D / 16);
  static constexpr int UK = KU / G::THREADS;
  static_assert(G::NSPLIT == 1, "paged source is single-split");
  static_assert(UK * G::THREADS == KU, "units");
  struct Stage {
    u32x4_t k[UK];
    u32x4_t v[UK];
  };

  // Physical block of the tile `it` (uniform): a scalar load from the block
  // table (read-only for the whole launch, so it may use the constant path).
  __device__ __forceinline__ int64_t tile_base(int it) const {
    const int last = (n_keys - 1) / G::BN;  // padding tiles reuse the last live block: always inside the table
    const unsigned key0 = (unsigned)(it < last ? it : last) * G::BN;
    const int32_t phys = bt[key0 / (unsigned)bs];
    return (int64_t)phys * blk_stride + head_off + (int64_t)(key0 % (unsigned)bs) * G::D;
  }

  // `base` is tile_base(it), computed one tile ahead by the caller.
  __device__ __forceinline__ void load(Stage &st, int it, int64_t base, unsigned tid) const {
    asm volatile("" : "+v"(tid));
    const unsigned key0 = (unsigned)it * G::BN;
    const uint8_t *kbase = kc + base, *vbase = vc + base;
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const unsigned t = u / (G::D / 16), c = u % (G::D / 16);
      const bool live = key0 + t < (unsigned)n_keys;
      st.k[j] = live ? ldg<u32x4_t>(kbase + (t * G::D + 16 * c)) : u32x4_t{0, 0, 0, 0};
      st.v[j] = live ? ldg<u32x4_t>(vbase + (t * G::D + 16 * c)) : u32x4_t{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(const Stage &st, char *stage, int tid) const {
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const int u = tid + j * G::THREADS;
      const int t = u / (G::D / 16), c = u % (G::D / 16);
      *reinterpret_cast<u32x4_t *>(stage + G::k_off(t, 2 * c)) = lo16(st.k[j]);
      *reinterpret_cast<u32x4_t *>(stage + G::k_off(t, 2 * c + 1)) = hi16(st.k[j]);
      char *vrow = stage + G::KT + t * G::VROW + 32 * c;
      *reinterpret_cast<u32x4_t *>(vrow) = lo16(st.v[j]);
      *reinterpret_cast<u32x4_t *>(vrow + 16) = hi16(st.v[j]);
    }
  }

  // fp8 bytes 0..7 / 8..15 of a unit -> 8 bf16 (exact)
  static __device__ __forceinline__ u32x4_t lo16(const u32x4_t &x) {
    return u32x4_t{e4m3x2_to_bf16x2<false>(x[0]), e4m3x2_to_bf16x2<true>(x[0]), e4m3x2_to_bf16x2<false>(x[1]),
                   e4m3x2_to_bf16x2<true>(x[1])};
  }
  static __device__ __forceinline__ u32x4_t hi16(const u32x4_t &x) {
    return u32x4_t{e4m3x2_to_bf16x2<false>(x[2]), e4m3x2_to_bf16x2<true>(x[2]), e4m3x2_to_bf16x2<false>(x[3]),
                   e4m3x2_to_bf16x2<true>(x[3])};
  }
};

// ------------------------------------------------------------------ core loop

template <class G>
struct WaveState {
  f32x16_t o[G::NT][G::MT];
  float m[G::NT], l[G::NT];  // m: running reference max, log2 units
};

// max / sum of a value with its partner lane (lane ^ 32) in one VALU op
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One key tile for one wave.  c = softmax_scale*log2(e) > 0.  `mask` (only
// read when HAS_MASK) is the additive key mask of this batch row, natural-log
// units; keys >= n_keys are removed.
template <class G, bool HAS_MASK>
__device__ __forceinline__ void compute_tile(WaveState<G> &ws, const u32x4_t (&qf)[G::NT][G::SD],
                                             const char *kt, const char *vt, int key0, int n_keys,
                                             float c, const float *mask, int lane) {
  asm volatile("" : "+v"(lane));  // lane-derived LDS offsets are recomputed per tile, not kept live
  const int l32 = lane & 31, h = lane >> 5;
  f32x16_t s[G::NT][G::KB];
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) s[nt][kb] = f32x16_t{};

  // QK^T: fragment f = sd*KB + kb feeds NT MFMAs.  All fragments are
  // written as loads up front; the scheduling groups below order them as
  // RA reads ahead, then (MFMA x NT, next read) pairs, so RA LDS reads stay in
  // flight behind the MFMAs while only RA+1 fragments are live.
  {
    constexpr int NF = G::SD * G::KB, RA = G::GRP < NF ? G::GRP : NF;
    // K fragment (kb, sd): row kb*32 + l32, chunk 2*sd + h.  The XOR swizzle
    // only touches the low 3 chunk bits, so the address is one of 4 per-lane
    // bases plus a compile-time offset.
    int kbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kbase[j] = l32 * (G::D * 2) + (((2 * j + h) ^ (l32 & 7)) << 4);
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t fb[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int kb = f % G::KB, sd = f / G::KB;
      fb[f] = *reinterpret_cast<const u32x4_t *>(kt + kbase[sd & 3] + kb * 32 * G::D * 2 + (sd >> 2) * 128);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt)
        s[nt][f % G::KB] = mfma32(as_bf16x8(fb[f]), as_bf16x8(qf[nt][f / G::KB]), s[nt][f % G::KB]);
    __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, G::NT, 0);
      if (f + RA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Scores into log2 units.  Without a mask the row max is taken on the raw
  // scores and the scale is folded into the exp2 argument (one FMA per score);
  // with a mask the scaled, masked score is formed first.
  if constexpr (HAS_MASK) {
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int key = key0 + kb * 32 + r4 * 8 + 4 * h;
        float mk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) mk[i] = key + i < n_keys ? mask[key + i] * kLog2e : -INFINITY;
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)  // removed keys stay -inf whatever their K holds
            s[nt][kb][4 * r4 + i] = mk[i] == -INFINITY ? -INFINITY : __builtin_fmaf(s[nt][kb][4 * r4 + i], c, mk[i]);
      }
  } else if (key0 + G::BN > n_keys) {  // ragged last tile (uniform branch)
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + kb * 32 + (v >> 2) * 8 + 4 * h + (v & 3);
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt)
          if (key >= n_keys) s[nt][kb][v] = -INFINITY;
      }
  }

  float mx[G::NT];
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mloc = __builtin_fmaxf(mloc, __builtin_fmaxf(s[nt][kb][v], s[nt][kb][v + 1]));
    mloc = pair_max(mloc);
    mx[nt] = HAS_MASK ? mloc : mloc * c;  // -inf * c = -inf (c > 0)
  }

  // Lazy rescale: the reference max m of a row only moves when the tile max
  // exceeds it by more than kTau (log2 units), so p = 2^(s - m) <= 2^kTau and
  // the O/l rescale (a VALU pass over every accumulator) is rare.  Exact: the
  // final O/l uses one consistent reference per row.
  bool grow = false;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) grow |= mx[nt] > ws.m[nt] + kTau;
  if (__ballot(grow) != 0) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      const float m_new = fmaxf(ws.m[nt], mx[nt]);
      const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(ws.m[nt] - m_new);
      ws.m[nt] = m_new;
      ws.l[nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] *= alpha;
    }
  }

  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  u32x4_t pb[G::NT][G::KB][2];
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const float m_use = ws.m[nt] == -INFINITY ? 0.0f : ws.m[nt];
    float lsum = ws.l[nt];
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s[nt][kb][v] = HAS_MASK ? fast_exp2(s[nt][kb][v] - m_use) : fast_exp2(__builtin_fmaf(s[nt][kb][v], c, -m_use));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // bit-cast plain scalars, never ext-vector elements: hipcc folded a
        // bit_cast of pb[..][i] to element 0 for every i
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = pack_bf16(s[nt][kb][8 * kk + 2 * i], s[nt][kb][8 * kk + 2 * i + 1]);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), ones, lsum, false);
        }
        pb[nt][kb][kk] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
    ws.l[nt] = lsum;
  }

  // PV: fragment f = (kb*2 + kk)*MT + mt, same read-ahead ordering.  The A
  // fragment (d rows mt*32 + l32, k-slots j = 0..7 of lane-half h) must hold
  // the keys that P's B fragment holds: kb*32 + 16kk + 8(j/4) + 4h + j%4.  Two
  // transposing reads (t = j/4) fetch it: in 16-lane group g the reading lane
  // 4m + j names the 8 bytes V[kb*32 + 16kk + 8t + 4h + j][mt*32 + 16(g%2) + 4m ..],
  // and output lane 16g + 4m + c receives element c of those four rows.
  {
    constexpr int NF = G::KB * 2 * G::MT, RA = G::GRP < NF ? G::GRP : NF;
    const int vlane = (4 * h + ((lane >> 2) & 3)) * G::VROW + (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t fb[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mt = f % G::MT, kk = (f / G::MT) % 2, kb = f / (2 * G::MT);
      const char *p = vt + vlane + (kb * 32 + kk * 16) * G::VROW + mt * 64;
      const u32x2_t a0 = lds_read_tr16(p), a1 = lds_read_tr16(p + 8 * G::VROW);
      fb[f] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mt = f % G::MT, kk = (f / G::MT) % 2, kb = f / (2 * G::MT);
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt)
        ws.o[nt][mt] = mfma32(as_bf16x8(fb[f]), as_bf16x8(pb[nt][kb][kk]), ws.o[nt][mt]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RA, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, G::NT, 0);
      if (f + RA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The pipelined key loop shared by both kernels.  PF register stages keep
// the global loads of the next PF tiles in flight while a tile is computed
// from one LDS stage and the next is written to the other.  The iteration
// count is padded to a multiple of PF (padding tiles are all-masked zeros),
// so the body unrolls over the register stages with static indices and the
// accumulators never meet a branch.  Returns with the LDS free (barrier
// passed).
template <class G, bool HAS_MASK, class Src>
__device__ __forceinline__ void flash_loop(WaveState<G> &ws, const Src &src, const u32x4_t (&qf)[G::NT][G::SD],
                                           char *smem, float c, const float *mask) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sp = wave / G::RG;
  const int n_tiles = (src.n_keys + G::BN - 1) / G::BN;
  const int n_iter = (n_tiles + G::NSPLIT - 1) / G::NSPLIT;
  const int n_pad = (n_iter + G::PF - 1) / G::PF * G::PF;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    ws.m[nt] = -INFINITY;
    ws.l[nt] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] = f32x16_t{};
  }
  if (n_iter <= 0) return;

  typename Src::Stage st[G::PF];
#pragma unroll
  for (int u = 0; u < G::PF; ++u) src.load(st[u], u, src.tile_base(u), tid);
  int64_t next_base = src.tile_base(G::PF);  // address base of the next tile to load, looked up one tile early
  src.store(st[0], smem, tid);
  __syncthreads();
  for (int it0 = 0; it0 < n_pad; it0 += G::PF) {
#pragma unroll
    for (int u = 0; u < G::PF; ++u) {
      const int it = it0 + u;
      // register stage u held tile `it`, already written to LDS: refill it
      if (it + G::PF < n_pad) {
        src.load(st[u], it + G::PF, next_base, tid);
        next_base = src.tile_base(it + G::PF + 1);
      }
      // A split whose tile index runs past the last tile computes on an
      // all-zero, fully masked tile (p = 0).
      const int ti = it * G::NSPLIT + sp;
      const char *base = smem + (it & 1) * G::STAGE + sp * G::SPLIT_BYTES;
      compute_tile<G, HAS_MASK>(ws, qf, base, base + G::KT, ti * G::BN, src.n_keys, c, mask, lane);
      if (it + 1 < n_pad) src.store(st[(u + 1) % G::PF], smem + ((it + 1) & 1) * G::STAGE, tid);
      __syncthreads();
    }
  }
}

// Merge the NSPLIT key-split partial states into the split-0 waves (LDS).
template <class G>
__device__ __forceinline__ void merge_splits(WaveState<G> &ws, char *smem) {
  if constexpr (G::NSPLIT > 1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % G::RG, sp = wave / G::RG;
    constexpr int NREG = G::NT * (G::MT * 16 + 2);
    float *red = reinterpret_cast<float *>(smem);
    static_assert((G::NSPLIT - 1) * G::RG * NREG * 64 * 4 <= G::LDS, "merge space");
    if (sp > 0) {
      float *dst = red + ((sp - 1) * G::RG + rg) * NREG * 64 + lane;
      int r = 0;
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        dst[(r++) * 64] = ws.m[nt];
        dst[(r++) * 64] = ws.l[nt];
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v) dst[(r++) * 64] = ws.o[nt][mt][v];
      }
    }
    __syncthreads();
    if (sp == 0) {
#pragma unroll
      for (int s = 1; s < G::NSPLIT; ++s) {
        const float *src = red + ((s - 1) * G::RG + rg) * NREG * 64 + lane;
        int r = 0;
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          const float m2 = src[(r++) * 64], l2 = src[(r++) * 64];
          const float M = fmaxf(ws.m[nt], m2);
          const float Mu = M == -INFINITY ? 0.0f : M;
          const float a1 = fast_exp2(ws.m[nt] - Mu), a2 = fast_exp2(m2 - Mu);
          ws.m[nt] = M;
          ws.l[nt] = ws.l[nt] * a1 + l2 * a2;
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) ws.o[nt][mt][v] = ws.o[nt][mt][v] * a1 + src[(r++) * 64] * a2;
        }
      }
    }
  }
}

// Linear workgroup id -> logical tile id, so that consecutive logical tiles
// (which share K/V) run on the same XCD: the hardware deals workgroups to the
// 8 XCDs round-robin.
__device__ __forceinline__ int xcd_remap(int lin, int total) {
  if (total % 8) return lin;
  return (lin % 8) * (total / 8) + lin / 8;
}

// A negative softmax scale is applied as a positive one on -q (exact), so the
// kernels only ever see c > 0.
__device__ __forceinline__ u32x4_t neg_bf16x8(u32x4_t x, uint32_t sign) {
  return u32x4_t{x[0] ^ sign, x[1] ^ sign, x[2] ^ sign, x[3] ^ sign};
}

// ------------------------------------------------------------------ encoder kernel

template <class G, bool F32IN, bool HAS_MASK>
__global__ __launch_bounds__(G::THREADS) __attribute__((amdgpu_waves_per_eu(G::WPE, G::WPE)))
void encoder_fwd_kernel(EncoderLaunch a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];  // G::LDS bytes
  const int n_qt = (a.Sq + G::BM - 1) / G::BM;
  const int total = n_qt * a.H * a.B;
  const int lid = xcd_remap(blockIdx.x, total);
  const int qt = lid % n_qt, h = (lid / n_qt) % a.H, b = lid / (n_qt * a.H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % G::RG, sp = wave / G::RG;
  const int l32 = lane & 31, hh = lane >> 5;
  constexpr int ES = F32IN ? 4 : 2;
  const uint32_t qsign = a.q_neg ? 0x80008000u : 0u;

  // Q fragments (B operand of S^T = K Q^T): row = lane%32, 8 d per lane-half
  u32x4_t qf[G::NT][G::SD];
  const char *qb = reinterpret_cast<const char *>(a.q) + (b * a.qs[0] + h * a.qs[1]) * ES;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int row = qt * G::BM + (rg * G::NT + nt) * 32 + l32;
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd) {
      const char *p = qb + (row * a.qs[2] + 16 * sd + 8 * hh) * ES;
      u32x4_t x = {0, 0, 0, 0};
      if (row < a.Sq) {
        if constexpr (F32IN) {
          const u32x4_t x0 = ldg<u32x4_t>(p), x1 = ldg<u32x4_t>(p + 16);
          x = u32x4_t{pack_bf16(__uint_as_float(x0[0]), __uint_as_float(x0[1])),
                      pack_bf16(__uint_as_float(x0[2]), __uint_as_float(x0[3])),
                      pack_bf16(__uint_as_float(x1[0]), __uint_as_float(x1[1])),
                      pack_bf16(__uint_as_float(x1[2]), __uint_as_float(x1[3]))};
        } else {
          x = ldg<u32x4_t>(p);
        }
      }
      qf[nt][sd] = neg_bf16x8(x, qsign);
    }
  }

  EncSrc<G, F32IN> src;
  src.kb = reinterpret_cast<const char *>(a.k) + (b * a.ks[0] + h * a.ks[1]) * ES;
  src.vb = reinterpret_cast<const char *>(a.v) + (b * a.vs[0] + h * a.vs[1]) * ES;
  src.ks = a.ks[2];
  src.vs = a.vs[2];
  src.kstep = (int64_t)G::NSPLIT * G::BN * a.ks[2] * ES;
  src.vstep = (int64_t)G::NSPLIT * G::BN * a.vs[2] * ES;
  src.n_keys = a.Skv;
  const float *mask = HAS_MASK ? a.mask + b * a.mask_sb : nullptr;
  src.mask = mask;

  WaveState<G> ws;
  flash_loop<G, HAS_MASK>(ws, src, qf, smem, a.c, mask);
  merge_splits<G>(ws, smem);
  if (sp != 0) return;

  const int HD = a.H * G::D;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int row = qt * G::BM + (rg * G::NT + nt) * 32 + l32;
    const float lt = pair_sum(ws.l[nt]);
    if (row >= a.Sq) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (a.lse && hh == 0)
      a.lse[((int64_t)b * a.H + h) * a.Sq + row] = lt > 0.0f ? (ws.m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = mt * 32 + r4 * 8 + 4 * hh;
        const f32x4_t val = {ws.o[nt][mt][4 * r4 + 0] * inv, ws.o[nt][mt][4 * r4 + 1] * inv,
                             ws.o[nt][mt][4 * r4 + 2] * inv, ws.o[nt][mt][4 * r4 + 3] * inv};
        if (a.out) {
          const int64_t off = b * a.os[0] + h * a.os[1] + row * a.os[2] + d0;
          if (a.out_f32) {
            *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.out) + off) = val;
          } else {
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<__bf16 *>(a.out) + off) =
                u32x2_t{pack_bf16(val[0], val[1]), pack_bf16(val[2], val[3])};
          }
        }
        if (a.res_out) {
          const int64_t off = ((int64_t)b * a.Sq + row) * HD + h * G::D + d0;
          const f32x4_t r = ldg<f32x4_t>(a.res + off);
          *reinterpret_cast<f32x4_t *>(a.res_out + off) = r + val;
        }
      }
  }
}

// ------------------------------------------------------------------ prefill kernel

template <class G>
__global__ __launch_bounds__(G::THREADS) __attribute__((amdgpu_waves_per_eu(G::WPE, G::WPE)))
void prefill_paged_kernel(PrefillLaunch a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];  // G::LDS bytes
  const int rows = a.G * a.Lq;  // packed (head, token) rows per KV head
  const int n_rt = (rows + G::BM - 1) / G::BM;
  const int lid = xcd_remap(blockIdx.x, n_rt * a.Hkv);
  const int rt = lid % n_rt, kvh = lid / n_rt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % G::RG;
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t row_base = (int64_t)kvh * rows;  // first packed row of this KV head in [Hq*Lq]
  const uint32_t qsign = a.q_neg ? 0x80008000u : 0u;

  u32x4_t qf[G::NT][G::SD];
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int r = rt * G::BM + (rg * G::NT + nt) * 32 + l32;
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd)
      qf[nt][sd] = neg_bf16x8(
          r < rows ? ldg<u32x4_t>(a.q + (row_base + r) * G::D + 16 * sd + 8 * hh) : u32x4_t{0, 0, 0, 0}, qsign);
  }

  PagedSrc<G> src;
  src.kc = a.kc;
  src.vc = a.vc;
  src.bt = (const __attribute__((address_space(4))) int32_t *)(a.bt);
  src.head_off = (int64_t)kvh * a.bs * G::D;
  src.blk_stride = (int64_t)a.Hkv * a.bs * G::D;
  src.bs = a.bs;
  src.n_keys = a.L_act;

  WaveState<G> ws;
  flash_loop<G, false>(ws, src, qf, smem, a.c, nullptr);

#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int r = rt * G::BM + (rg * G::NT + nt) * 32 + l32;
    const float lt = pair_sum(ws.l[nt]);
    if (r >= rows) continue;
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    if (a.lse && hh == 0) a.lse[row_base + r] = lt > 0.0f ? (ws.m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = mt * 32 + r4 * 8 + 4 * hh;
        *reinterpret_cast<u32x2_t *>(a.out + (row_base + r) * G::D + d0) =
            u32x2_t{pack_bf16(ws.o[nt][mt][4 * r4 + 0] * inv, ws.o[nt][mt][4 * r4 + 1] * inv),
                    pack_bf16(ws.o[nt][mt][4 * r4 + 2] * inv, ws.o[nt][mt][4 * r4 + 3] * inv)};
      }
  }
}

// ------------------------------------------------------------------ launchers

using EncGeo = Geo<64, 64, 1, 4, 2, 4, 2>;     // BM 128, 8 waves, 2 key splits, 2 tiles in flight
using EncGeoF32 = Geo<64, 64, 1, 4, 2, 4, 1>;  // fp32 inputs: twice the staging registers per tile
using PrefGeo = Geo<256, 32, 1, 8, 1, 2, 1>;   // BM 256, 8 waves of 32 rows, 2 waves per SIMD

// Launch with G::LDS bytes of dynamic LDS; kernels above 64 KiB are opted in
// once per process (hipFuncSetAttribute is per function, not per device).
template <class G, class K, class A>
hipError_t launch_lds(K kernel, dim3 grid, const A &a, hipStream_t stream) {
  if constexpr (G::LDS > 65536) {
    static const hipError_t opt =
        hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    if (opt != hipSuccess) return opt;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(G::THREADS), G::LDS, stream, a);
  return hipGetLastError();
}

hipError_t launch_encoder(const EncoderLaunch &a, bool f32_in, hipStream_t stream) {
  const int n_qt = (a.Sq + EncGeo::BM - 1) / EncGeo::BM;
  const dim3 grid(n_qt * a.H * a.B);
  static_assert(EncGeo::BM == EncGeoF32::BM && EncGeo::THREADS == EncGeoF32::THREADS, "same launch shape");
  if (f32_in)
    return a.mask ? launch_lds<EncGeoF32>(encoder_fwd_kernel<EncGeoF32, true, true>, grid, a, stream)
                  : launch_lds<EncGeoF32>(encoder_fwd_kernel<EncGeoF32, true, false>, grid, a, stream);
  return a.mask ? launch_lds<EncGeo>(encoder_fwd_kernel<EncGeo, false, true>, grid, a, stream)
                : launch_lds<EncGeo>(encoder_fwd_kernel<EncGeo, false, false>, grid, a, stream);
}

int encoder_rows_per_block() { return EncGeo::BM; }

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream) {
  const int rows = a.G * a.Lq;
  const int n_rt = (rows + PrefGeo::BM - 1) / PrefGeo::BM;
  return launch_lds<PrefGeo>(prefill_paged_kernel<PrefGeo>, dim3(n_rt * a.Hkv), a, stream);
}

int prefill_key_tile() { return PrefGeo::BN; }

}  // namespace mi355
