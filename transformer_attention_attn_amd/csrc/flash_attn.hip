// Tiled online-softmax ("flash") attention forward for gfx950.
//
// Two key loops serve three kernels: flash_loop stages K/V tiles through
// registers (fp32 or masked encoder inputs, the prefill without a
// workspace); flash_loop_dma copies them straight into LDS with direct
// global -> LDS loads (the bf16 encoder, the prefill over bf16 tile images).
// The kernels:
//   * the non-causal encoder (q/k/v [B,H,S,D] bf16 or fp32, optional additive
//     key mask, optional RoPE on the Q rows, fused residual-add epilogue);
//   * the history-only GQA prefill over a paged FP8 (e4m3fn) KV cache, whose
//     G query heads per KV head are packed into the M dimension (rows r of a KV
//     head are (head g, token t) with r = g*Lq + t);
//   * causal attention over the current tokens' bf16 K/V, launched after the
//     history prefill: that kernel hands over its normalised fp32 output and
//     lse per row, and this one resumes the online softmax from them, which
//     is the log-sum-exp merge of the two parts.
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
// 32*NT rows; its Q fragments stay on chip for the whole loop, in registers
// except the first Geo::QL, which sit in LDS.
//
// Per key tile (BN keys), per wave:
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, query rows on N), so
//   every lane owns one query row (lane % 32) and 16 keys per 32-key block;
//   row max: in-lane max + one v_permlane32_swap with the partner lane (the
//   bf16 encoder skips it while a row's half-tile sums stay below 2^kTau:
//   Geo::LAZYSUM);
//   P = exp2(S*c - m) with the scale folded into one FMA (c > 0, log2 units),
//   packed to bf16 straight into the B operand of O^T += V^T P^T (d on M,
//   rows on N): P never leaves registers; the row sum is taken on the packed
//   bf16 P with v_dot2_f32_bf16, so it normalises exactly the values that were
//   multiplied into V.
//
// Software pipeline: K tiles sit one tile ahead of V tiles in LDS, so while a
// wave's MFMAs compute S for tile i+1, its VALU runs the softmax of tile i;
// then the PV MFMAs of tile i run while the staged global loads are written
// to LDS and the next ones are issued.  One barrier per tile.
//
// LDS: K and V tiles as [key][d] with padded rows, V read as the A operand
// of the PV MFMA (d on M, keys on K) with ds_read_b64_tr_b16.  The pads make
// the 16-byte K reads, the transposing V reads and the 16-byte writes all
// bank-conflict-free while every fragment address stays one per-lane base
// plus an immediate.  (Tile images copied by DMA hold K chunk-major and V
// transposed instead: see Geo.)  Global K/V loads are raw buffer loads whose
// range ends at the last valid key, so out-of-range keys read as zeros
// without a branch.
#include "device_common.h"
#include "launch.h"

namespace mi355 {

constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units
constexpr float kSumTrig = 256.0f;      // 2^kTau: a half-tile row sum above it may need a new reference
constexpr float kFloatMax = __FLT_MAX__;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family: 32-bit data format, no swizzle)

// Raw buffer resource over [base, base + bytes).  Both are uniform at every
// call; readfirstlane makes that visible to the compiler, which otherwise may
// compute them in vector registers and wrap each load in a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}
// 16 bytes at byte offset `off`; zeros when the range check fails
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int D_, int BN_, int NT_, int RG_, int NSPLIT_, int GRP_, int OCC_, bool VFIRST_ = false, int QL_ = 0,
          bool PVPRIO_ = false, bool DMA_ = false, bool EDMA_ = false, bool RARE_ALPHA_ = false,
          bool LAZYSUM_ = false>
struct Geo {
  static constexpr int D = D_, BN = BN_, NT = NT_, RG = RG_, NSPLIT = NSPLIT_;
  static constexpr int GRP = GRP_;  // LDS fragments read ahead of the MFMAs that use them
  static constexpr int WPE = OCC_;  // waves per SIMD the kernel is compiled for (register budget 512 / WPE)
  // Slot order of the pipelined phases: VALU slice before the slot's MFMA
  // (hides the fragment read latency behind the VALU; best when the VALU work
  // per MFMA is large, D = 64) or after it (best at D = 256).
  static constexpr bool VFIRST = VFIRST_;
  static constexpr int WAVES = RG * NSPLIT, THREADS = 64 * WAVES;
  static constexpr int BM = 32 * NT * RG;
  // K rows: D bf16 + one 16-byte pad chunk, so 16 consecutive rows start in 16
  // different 16-byte bank groups.  V rows: D bf16, plus 64 bytes after every
  // row (D >= 128) or every second row (D = 64), so the 4 consecutive rows one
  // transposing read touches start in 4 different 64-byte bank groups.
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VSH = (D * 2) % 256 == 0 ? 0 : 1;
  // DMA: tiles arrive as ready-made bf16 images copied global -> LDS by
  // direct loads (1 KB per wave instruction, no registers, no conversion).
  // A direct load cannot pad inside its 1 KB, so K is chunk-major instead of
  // padded: the 16-byte chunk c (d = 8c .. 8c+7) of key k sits at
  // c*BN*16 + k*16, which keeps the 32 keys one fragment read touches in 512
  // contiguous bytes.  V is stored transposed (V^T), so that a PV A fragment
  // (d = lane%32, 8 keys) is one 16-byte read instead of two 8-byte
  // transposing reads: each k-step's 16 keys fill one half of the image, a
  // 32-byte row per d (vt_off), so the k-step and the d tile are immediate
  // offsets; within a row the two 16-byte chunks swap on d bit 2 ^ bit 3,
  // which puts 8 (and 16) consecutive lanes in 8 (and 16) different 16-byte
  // bank groups.  Three buffers per operand let a tile's copy run two
  // iterations ahead of its use.
  static constexpr bool DMA = DMA_;
  // EDMA: the caller's bf16 K and V rows copied global -> LDS by the same
  // direct loads (no image pass): K chunk-major as above, V row-major with
  // the two 64-byte halves of a row swapped when key bit 1 is set
  // (v_frag_edma), which stands in for the padding a direct load cannot make.
  static constexpr bool EDMA = EDMA_;
  static constexpr bool LINEAR = DMA || EDMA;  // tiles land unpadded, K chunk-major
  // RARE_ALPHA: phase A hands out the rescale exponent and the caller takes
  // its exp2 on the rare path where some row's reference moved, instead of
  // one exp2 per row and tile on the common path; the tile's row sum then
  // starts from zero and joins l at the end of the step.  Carrying both
  // across the phases costs registers (kept off where the key loop would
  // spill).
  static constexpr bool RARE_ALPHA = RARE_ALPHA_;
  // LAZYSUM (with RARE_ALPHA): no row max on the common path.  While a row's
  // reference holds, every p = 2^(s c - m) is at most 2^kTau, so a half
  // tile's row sum (which the dot2s take anyway) above 2^kTau is a
  // conservative sign that it may have to move: only then is the tile max
  // taken, the reference moved and the half's P recomputed (same bits for
  // the rows that keep their reference).  Phase A checks the first half
  // before the PV MFMAs use it, phase B the second half before its MFMAs.
  static constexpr bool LAZYSUM = LAZYSUM_;
  static constexpr int NBUF = LINEAR ? 3 : 2;
  static constexpr int KTILE = LINEAR ? BN * D * 2 : BN * KROW;
  static constexpr int VTILE = LINEAR ? BN * D * 2 : BN * D * 2 + (BN >> VSH) * 64;
  static constexpr int KSLOT = NSPLIT * KTILE;                    // one K buffer: every split's tile
  // one V buffer, then the tiles' staged key mask (none over direct copies)
  static constexpr int VSLOT = NSPLIT * VTILE + (EDMA ? 0 : NSPLIT * BN * 4);
  static constexpr int KB = BN / 32;  // 32-key blocks per tile
  static constexpr int SD = D / 16;   // k-steps of the QK^T contraction
  static constexpr int MT = D / 32;   // d tiles of O^T
  static constexpr int NFQ = SD * KB, NFV = 2 * KB * MT;  // LDS fragments per tile: QK, PV
  static constexpr int MERGE = (NSPLIT - 1) * RG * NT * (MT * 16 + 2) * 64 * 4;  // split partials (merge_splits)
  // The first QL Q fragments of every lane live in LDS, not in registers: one
  // 16-byte slot per (fragment, row block, thread) after the K/V buffers.
  // Read with ds_read they wait on the LDS counter only; a register spilled
  // instead would be reloaded from scratch, and that wait (the vector memory
  // counter, in order) also drains the K/V tile loads in flight.
  static constexpr int QL = QL_;
  // Raise the wave's issue priority around each PV MFMA: with two waves per
  // SIMD, a wave whose PV MFMA is ready then wins the arbiter over the other
  // wave's softmax VALU, and the matrix pipe idles less (prefill ~1% faster;
  // the VALU-bound encoder gains nothing).
  static constexpr bool PVPRIO = PVPRIO_;
  static constexpr int QOFF = NBUF * (KSLOT + VSLOT) > MERGE ? NBUF * (KSLOT + VSLOT) : MERGE;
  // EDMA: the tile's fp32 residual rows (BM x D), copied to LDS with the first
  // K/V tiles and read by the epilogue (ResRows); apart from buffers and merge
  // space.  At D = 64 the whole geometry takes 80 KiB: two workgroups per CU.
  static constexpr int RES = EDMA ? BM * D * 4 : 0;
  static constexpr int LDS = QOFF + QL * NT * THREADS * 16 + RES;  // buffers (or merge space), Q slots, residual
  // softmax VALU instructions issued between consecutive QK MFMA groups
  static constexpr int VPM = (NT * (7 * BN / 4 + 8) + NFQ - 1) / NFQ;
  static_assert(D % 64 == 0 && BN % 32 == 0 && (VSH == 0 || D == 64), "tile shape");
  static_assert(QL >= 0 && QL <= SD, "Q fragments in LDS");
  static_assert(!DMA || (NSPLIT == 1 && BN == 32 && KTILE % 1024 == 0 && VTILE % 1024 == 0),
                "tile images: one key split, 32-key tiles, 1 KB pieces");
  static_assert(!EDMA || (!DMA && D == 64 && BN % 32 == 0 && QL == 0 && KSLOT % (1024 * WAVES) == 0),
                "direct encoder tiles: 128-byte rows, 32-key blocks, whole rounds of 1 KB pieces");
  static_assert(LDS <= 160 * 1024, "LDS budget (gfx950: 160 KiB per workgroup)");

  static __device__ __forceinline__ int k_row(int key) { static_assert(!LINEAR, "padded K rows"); return key * KROW; }
  // byte offset of this lane's first QK fragment (key lane%32, chunk lane/32)
  // and of fragment (32-key block kb, k-step sd) relative to it
  static __device__ __forceinline__ int k_lane(int lane) {
    return LINEAR ? (lane & 31) * 16 + (lane >> 5) * BN * 16 : (lane & 31) * KROW + 16 * (lane >> 5);
  }
  static constexpr int k_frag(int kb, int sd) { return LINEAR ? kb * 512 + sd * 2 * BN * 16 : kb * 32 * KROW + 32 * sd; }
  static __device__ __forceinline__ int v_row(int key) { return key * (D * 2) + (key >> VSH) * 64; }
  // DMA: the V^T chunk of (d, k-step kk, lane half h) holds, as elements
  // j = 0..7, the keys 16kk + 8(j/4) + 4h + j%4 (the key order of P's B
  // fragment) and sits at vt_off(d, kk, h).
  static __host__ __device__ constexpr int vt_swz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }
  static __host__ __device__ constexpr int vt_off(int d, int kk, int h) {
    return kk * D * 32 + d * 32 + 16 * (h ^ vt_swz(d));
  }
  static __host__ __device__ constexpr int vt_key(int kk, int h, int j) { return 16 * kk + 8 * (j >> 2) + 4 * h + (j & 3); }
};

// ------------------------------------------------------------------ sources
//
// A source loads the K and V tiles of iteration `it` (every split's tile,
// keys it*NSPLIT*BN ...) into a register stage and writes them to an LDS
// buffer.  Keys past n_keys read as zeros (buffer range check).

// Rotary position embedding (vit-encoder-neuron-kernels, "Kernels"): pair k
// of token s turns by the angle of the tables' (cos[s,k], sin[s,k]); pairing
// 1 ("half") pairs lane k with lane k + D/2, pairing 2 ("interleaved") lane
// 2k with lane 2k + 1.  For a pair (a, b): a' = a cos - b sin,
// b' = b cos + a sin, in fp32, rounded to bf16 afterwards.
__device__ __forceinline__ void rot_pair(float &a, float &b, float c, float s) {
  const float a2 = __builtin_fmaf(-b, s, a * c);
  b = __builtin_fmaf(a, s, b * c);
  a = a2;
}

// 8 raw elements (bf16: one u32x4; fp32: two) <-> fp32
template <bool F32>
__device__ __forceinline__ void unpack8(const u32x4_t (&x)[F32 ? 2 : 1], float (&f)[8]) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(x[i / 4][i % 4]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(x[0][i]);
      f[2 * i + 1] = bf16_hi(x[0][i]);
    }
  }
}
__device__ __forceinline__ u32x4_t pack8(const float (&f)[8]) {
  return u32x4_t{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
}

// Encoder K/V: [B,H,S_kv,D] strided, bf16 or fp32 (fp32 rounded to bf16 on
// the LDS write).  A unit is 8 elements of one key; unit u of an iteration is
// key (u / KU)*BN + (u % KU)/(D/8) of the iteration, chunk u % (D/8).
template <class G, bool F32, bool HAS_MASK>
struct EncSrc {
  const char *kb, *vb;    // this (b,h)'s K and V base
  const float *mask;      // this batch row's additive mask (HAS_MASK)
  int64_t kstep, vstep;   // bytes per iteration (NSPLIT*BN keys)
  uint32_t krow, vrow;    // bytes between consecutive keys
  int n_keys;
  static constexpr int ES = F32 ? 4 : 2;
  static constexpr int W = F32 ? 2 : 1;  // 16-byte loads per unit
  static constexpr int CPR = G::D / 8;   // units per key row
  static constexpr int KU = G::BN * CPR;
  static constexpr int KEYS = G::NSPLIT * G::BN;
  static constexpr int UK = KEYS * CPR / G::THREADS;
  static_assert(UK >= 1 && UK * G::THREADS == KEYS * CPR, "units");
  static_assert(KEYS <= G::THREADS, "mask staging: one key per thread");
  static_assert(KEYS <= 128, "records(): KEYS * row bytes must stay below 2^31 (row < 2^24 bytes)");
  struct Stage {
    u32x4_t k[UK][W], v[UK][W];
    float vm[UK];  // mask value of each V unit's key
    float m;       // mask value of key tid % KEYS
  };

  static __device__ __forceinline__ unsigned key_of(unsigned u) { return (u / KU) * G::BN + (u % KU) / CPR; }
  static __device__ __forceinline__ unsigned chunk_of(unsigned u) { return u % CPR; }

  // bytes of the iteration's keys that exist (the key stride is below 2^24
  // bytes, checked on the host).  A select on the uniform iteration index
  // against loop-invariant bounds keeps this on the scalar unit (a clamp
  // compiles to a vector med3 and a vector multiply).
  __device__ __forceinline__ uint32_t records(int it, uint32_t row) const {
    const int full = n_keys / KEYS;  // iterations whose keys all exist
    const uint32_t n = it < full ? (uint32_t)KEYS : it == full ? (uint32_t)(n_keys % KEYS) : 0u;
    return n * row;
  }
  __device__ __forceinline__ int64_t tile_base(int) const { return 0; }

  __device__ __forceinline__ void load_k(Stage &st, int it, int64_t, unsigned tid) const {
    const auto r = make_rsrc(kb + it * kstep, records(it, krow));
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const uint32_t off = key_of(u) * krow + chunk_of(u) * (8 * ES);
#pragma unroll
      for (int x = 0; x < W; ++x) st.k[j][x] = buf_load16(r, off + 16 * x);
    }
  }
  __device__ __forceinline__ void load_v(Stage &st, int it, int64_t, unsigned tid) const {
    const auto r = make_rsrc(vb + it * vstep, records(it, vrow));
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const uint32_t off = key_of(u) * vrow + chunk_of(u) * (8 * ES);
#pragma unroll
      for (int x = 0; x < W; ++x) st.v[j][x] = buf_load16(r, off + 16 * x);
    }
    if constexpr (HAS_MASK) {
      const auto rm = make_rsrc(mask + (int64_t)it * KEYS, records(it, 4));
#pragma unroll
      for (int j = 0; j < UK; ++j) st.vm[j] = buf_load_f32(rm, key_of(tid + j * G::THREADS) * 4);
      st.m = buf_load_f32(rm, (tid % KEYS) * 4);
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

  __device__ __forceinline__ void store_k(const Stage &st, char *slot, unsigned tid) const {
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const unsigned t = (u % KU) / CPR;
      const u32x4_t x = to_bf16(st.k[j]);
      *reinterpret_cast<u32x4_t *>(slot + (u / KU) * G::KTILE + G::k_row(t) + 16 * chunk_of(u)) = x;
    }
  }
  // V rows of keys the mask removes are written as zeros (p = 0 there, and a
  // non-finite V must not turn 0 * V into NaN); the staged mask is in log2
  // units, -inf for removed keys and keys past n_keys.
  __device__ __forceinline__ void store_v(const Stage &st, char *slot, int it, unsigned tid) const {
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const unsigned t = (u % KU) / CPR;
      u32x4_t x = to_bf16(st.v[j]);
      if constexpr (HAS_MASK) x = st.vm[j] == -INFINITY ? u32x4_t{0, 0, 0, 0} : x;
      *reinterpret_cast<u32x4_t *>(slot + (u / KU) * G::VTILE + G::v_row(t) + 16 * chunk_of(u)) = x;
    }
    if constexpr (HAS_MASK) {
      // every thread writes key tid % KEYS (identical values where threads coincide)
      const unsigned t = tid % KEYS;
      const bool live = it * KEYS + (int)t < n_keys && st.m != -INFINITY;
      reinterpret_cast<float *>(slot + G::NSPLIT * G::VTILE)[t] = live ? st.m * kLog2e : -INFINITY;
    }
  }
};

// Paged FP8 K/V: cache [num_blocks, Hkv, bs, D] e4m3fn.  A unit is 8 fp8 of
// each half of one key row: lane i of a row's D/16 lanes takes bytes
// [8i, 8i+8) and [D/2 + 8i, D/2 + 8i + 8), so that in LDS (bf16, converted
// exactly) consecutive lanes write consecutive 16-byte chunks.  A tile (BN
// keys) never straddles a cache block (bs is a multiple of BN).
template <class G>
struct PagedSrc {
  const uint8_t *kc, *vc;
  const __attribute__((address_space(4))) int32_t *bt;  // constant address space: scalar loads
  int64_t head_off;    // kvh * bs * D
  int64_t blk_stride;  // Hkv * bs * D
  int bs, n_keys;
  static constexpr int LPR = G::D / 16;  // lanes per key row
  static constexpr int KU = G::BN * LPR;
  static constexpr int UK = KU / G::THREADS;
  static_assert(G::NSPLIT == 1, "paged source is single-split");
  static_assert(UK >= 1 && UK * G::THREADS == KU, "units");
  struct Stage {
    u32x2_t k[UK][2], v[UK][2];
  };

  // Byte offset of tile `it` in a cache (uniform): a scalar load from the
  // block table (read-only for the whole launch, so it may use the constant
  // path).  Tiles past the last live one reuse its block, so the lookup stays
  // inside the table; their loads read nothing (zero range).
  __device__ __forceinline__ int64_t tile_base(int it) const {
    const int last = (n_keys - 1) / G::BN;
    const unsigned key0 = (unsigned)(it < last ? it : last) * G::BN;
    const int32_t phys = bt[key0 / (unsigned)bs];
    return (int64_t)phys * blk_stride + head_off + (int64_t)(key0 % (unsigned)bs) * G::D;
  }
  __device__ __forceinline__ uint32_t records(int it) const {  // scalar select, as EncSrc::records
    const int full = n_keys / G::BN;
    const uint32_t n = it < full ? (uint32_t)G::BN : it == full ? (uint32_t)(n_keys % G::BN) : 0u;
    return n * G::D;
  }
  static __device__ __forceinline__ u32x2_t load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
  __device__ __forceinline__ void load(u32x2_t (&x)[UK][2], const uint8_t *cache, int it, int64_t base,
                                       unsigned tid) const {
    const auto r = make_rsrc(cache + base, records(it));
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      const uint32_t off = (u / LPR) * G::D + (u % LPR) * 8;
      x[j][0] = load8(r, off);
      x[j][1] = load8(r, off + G::D / 2);
    }
  }
  __device__ __forceinline__ void load_k(Stage &st, int it, int64_t base, unsigned tid) const {
    load(st.k, kc, it, base, tid);
  }
  __device__ __forceinline__ void load_v(Stage &st, int it, int64_t base, unsigned tid) const {
    load(st.v, vc, it, base, tid);
  }

  // 8 fp8 -> 8 bf16 (exact)
  static __device__ __forceinline__ u32x4_t cvt8(const u32x2_t &x) {
    return u32x4_t{e4m3x2_to_bf16x2<false>(x[0]), e4m3x2_to_bf16x2<true>(x[0]), e4m3x2_to_bf16x2<false>(x[1]),
                   e4m3x2_to_bf16x2<true>(x[1])};
  }
  __device__ __forceinline__ void store_k(const Stage &st, char *slot, unsigned tid) const {
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      char *p = slot + G::k_row(u / LPR) + 16 * (u % LPR);
      *reinterpret_cast<u32x4_t *>(p) = cvt8(st.k[j][0]);
      *reinterpret_cast<u32x4_t *>(p + G::D) = cvt8(st.k[j][1]);
    }
  }
  __device__ __forceinline__ void store_v(const Stage &st, char *slot, int, unsigned tid) const {
#pragma unroll
    for (int j = 0; j < UK; ++j) {
      const unsigned u = tid + j * G::THREADS;
      char *p = slot + G::v_row(u / LPR) + 16 * (u % LPR);
      *reinterpret_cast<u32x4_t *>(p) = cvt8(st.v[j][0]);
      *reinterpret_cast<u32x4_t *>(p + G::D) = cvt8(st.v[j][1]);
    }
  }
};

// Wait until at most N of this wave's vector memory operations are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Tile images of a KV head's history (G::DMA): tile t holds the K image
// (chunk-major, G::KTILE bytes) then the V^T image (G::VTILE
// bytes), each exactly as the key loop's LDS buffers hold them, so a tile is
// copied global -> LDS by direct buffer loads: 1 KB per wave instruction,
// lane L's 16 bytes at LDS base + 16 L.  Wave w issues pieces w, w + WAVES,
// ...  A tile at or past n_tiles gets an empty range and reads as zeros
// (the range check alone decides: the piece offset is an SGPR, the lane
// offset a VGPR inside the piece).
template <class G>
struct TileImgSrc {
  static constexpr int TIMG = G::KTILE + G::VTILE;
  static constexpr int KP = G::KTILE / 1024, VP = G::VTILE / 1024;  // 1 KB pieces
  const char *img;  // this KV head's first tile
  int n_tiles, n_keys;
  // pieces one wave issues per tile step (for its memory-counter waits)
  static constexpr int pieces(int wave) {
    return (KP + G::WAVES - 1 - wave) / G::WAVES + (VP + G::WAVES - 1 - wave) / G::WAVES;
  }
  static constexpr int PMAX = pieces(0), PMIN = pieces(G::WAVES - 1);
  static_assert(PMAX - PMIN <= 2, "wait_step covers three counts");
  // wait until at most this wave's pieces of one tile step are in flight
  static __device__ __forceinline__ void wait_step(int wave) {
    const int pw = pieces(wave);
    if (pw == PMAX) wait_vm<PMAX>();
    else if (pw == PMAX - 1) wait_vm<(PMAX - 1 >= 0 ? PMAX - 1 : 0)>();
    else wait_vm<(PMAX - 2 >= 0 ? PMAX - 2 : 0)>();
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile(int t) const {
    return make_rsrc(img + (int64_t)(t < n_tiles ? t : 0) * TIMG, t < n_tiles ? (uint32_t)TIMG : 0u);
  }
  static __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t r, char *dst, int first, int n, int wave,
                                              int lane) {
#pragma unroll
    for (int j = 0; j < (n + G::WAVES - 1) / G::WAVES; ++j) {
      const int piece = wave + j * G::WAVES;
      if ((j + 1) * G::WAVES <= n || piece < n)  // the test folds away for whole rounds of pieces
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + piece * 1024), 16,
                                                 lane * 16, first + piece * 1024, 0, 0);
    }
  }
  __device__ __forceinline__ void copy_k(char *dst, int t, int wave, int lane) const {
    copy(tile(t), dst, 0, KP, wave, lane);
  }
  __device__ __forceinline__ void copy_v(char *dst, int t, int wave, int lane) const {
    copy(tile(t), dst, G::KTILE, VP, wave, lane);
  }
};

// The encoder's K and V tiles copied global -> LDS by direct loads (G::EDMA;
// bf16 rows whose base and stride are multiples of 16 bytes, checked on the
// host).  An iteration's NSPLIT tiles of each operand are KSLOT / 1 KB pieces
// and wave w copies pieces w, w + WAVES, ...; piece p belongs to split p / PT,
// keys of that split's tile:
//   K: lane L takes element u = 64 (p % PT) + L of the tile's chunk-major
//      order, chunk c = u / BN (d = 8c .. 8c + 7) of key u % BN, which lands
//      at c * BN * 16 + key * 16;
//   V: lane L lands at byte 16 L of the piece, key 8 (p % PT) + L / 8,
//      physical chunk L % 8, and takes the key's logical chunk
//      (L % 8) ^ (4 * key bit 1) (the half swap v_frag_edma undoes).
// Each iteration's keys form one buffer range (as EncSrc's), so keys past
// n_keys read as zeros.
template <class G>
struct EncDmaSrc {
  static constexpr int PT = G::KTILE / 1024;            // pieces per split tile
  static constexpr int PW = G::KSLOT / 1024 / G::WAVES;  // pieces per wave and operand
  static constexpr int KEYS = G::NSPLIT * G::BN;
  static constexpr bool kNoScalarLoads = true;
  const char *kb, *vb;     // this (b,h)'s K and V base
  int64_t kstep, vstep;    // bytes per iteration
  uint32_t krow, vrow;     // bytes between consecutive keys
  int n_keys;
  uint32_t koff[PW], voff[PW];  // this lane's source offsets inside an iteration's keys

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int p = wave + j * G::WAVES, sp = p / PT, pp = p % PT;
      const int u = 64 * pp + lane, ck = u / G::BN, kk = u % G::BN;
      koff[j] = (uint32_t)(sp * G::BN + kk) * krow + ck * 16;
      const int kv = 8 * pp + (lane >> 3), cv = (lane & 7) ^ (((kv >> 1) & 1) << 2);
      voff[j] = (uint32_t)(sp * G::BN + kv) * vrow + cv * 16;
    }
  }
  __device__ __forceinline__ uint32_t records(int it, uint32_t row) const {
    const int full = n_keys / KEYS;
    const uint32_t n = it < full ? (uint32_t)KEYS : it == full ? (uint32_t)(n_keys % KEYS) : 0u;
    return n * row;
  }
  // wait until at most this wave's copies of one tile step are in flight
  static __device__ __forceinline__ void wait_step(int) { wait_vm<2 * PW>(); }
  __device__ __forceinline__ void copy_k(char *dst, int it, int wave, int) const {
    const auto r = make_rsrc(kb + it * kstep, records(it, krow));
#pragma unroll
    for (int j = 0; j < PW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + (wave + j * G::WAVES) * 1024),
                                               16, koff[j], 0, 0, 0);
  }
  __device__ __forceinline__ void copy_v(char *dst, int it, int wave, int) const {
    const auto r = make_rsrc(vb + it * vstep, records(it, vrow));
#pragma unroll
    for (int j = 0; j < PW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + (wave + j * G::WAVES) * 1024),
                                               16, voff[j], 0, 0, 0);
  }
};

// The fp32 residual rows of an encoder tile (BM rows x D columns of the
// token-major [B, Sq, H*D] stream) copied global -> LDS by direct loads
// (G::EDMA): 1 KB pieces of 4 rows, wave w copying pieces w, w + WAVES, ...
// Row r's 16-byte chunk c lands at r*D*4 + 16*(c ^ (r % 16)), so that the
// epilogue's reads (32 consecutive rows, one chunk) spread over the banks.
// Rows past the tile's nrows fall outside the buffer range and read as zeros;
// every offset is in the lane's VGPR, where the range check sees it.
template <class G>
struct ResRows {
  static __device__ __forceinline__ void copy(const float *tile, int nrows, int hidden, char *dst, int wave,
                                              int lane) {
    static_assert(G::D * 4 == 256 && (4 * G::WAVES) % 16 == 0 && (G::BM / 4) % G::WAVES == 0, "residual pieces");
    const uint32_t stride = (uint32_t)hidden * 4;
    const auto r = make_rsrc(tile, nrows > 0 ? (uint32_t)(nrows - 1) * stride + G::D * 4 : 0u);
    const int row = 4 * wave + (lane >> 4);  // row of piece `wave`; later pieces add 4 * WAVES rows
    const uint32_t off = (uint32_t)row * stride + 16 * ((lane & 15) ^ (row & 15));
#pragma unroll
    for (int j = 0; j < G::BM / 4 / G::WAVES; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void *)(dst + (wave + j * G::WAVES) * 1024), 16,
          off + (uint32_t)(j * 4 * G::WAVES) * stride, 0, 0, 0);
  }
  // byte offset of columns d0 .. d0 + 3 (d0 a multiple of 4) of tile row `row`
  static __device__ __forceinline__ int offset(int row, int d0) {
    return row * (G::D * 4) + 16 * ((d0 >> 2) ^ (row & 15));
  }
  // those columns as copy left them
  static __device__ __forceinline__ f32x4_t read(const char *src, int row, int d0) {
    return *reinterpret_cast<const f32x4_t *>(src + offset(row, d0));
  }
};

// Workgroup barrier without a memory fence: finishes this wave's LDS
// operations and meets the other waves.  A __syncthreads() here would also
// wait for the tile copies still in flight (a direct load counts as an LDS
// store), which must keep running across the barrier; their completion is
// waited for explicitly (wait_vm) before the barrier that publishes them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ per-tile pieces

template <class G>
struct WaveState {
  f32x16_t o[G::NT][G::MT];
  float m[G::NT], l[G::NT];  // m: running reference max, log2 units
  // G::RARE_ALPHA: the exponents' reference (m, or the lowest float while m =
  // -inf) and the raw tile max above which m moves ((m + kTau) / c, -inf while
  // m = -inf), both changed only when m does
  float mu[G::RARE_ALPHA ? G::NT : 1], thr[G::RARE_ALPHA ? G::NT : 1];
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

// S^T of one tile: s[nt][kb] = K-block kb . Q^T.  K fragment (kb, sd) is the
// 16 bytes at d = 16*sd + 8*(lane/32) of row kb*32 + lane%32.
// Q fragment (nt, sd): from LDS for sd < QL (qa: this thread's first slot),
// else from the registers.
template <class G>
__device__ __forceinline__ u32x4_t q_lds(const char *qa, int nt, int sd) {
  return *reinterpret_cast<const u32x4_t *>(qa + (sd * G::NT + nt) * G::THREADS * 16);
}
// Store the LDS-resident Q fragments of this thread into its slots (qa, as
// q_lds reads them; only this thread reads them back, so no barrier).
template <class G>
__device__ __forceinline__ void q_to_lds(const u32x4_t (&qf)[G::NT][G::SD], char *qa) {
#pragma unroll
  for (int sd = 0; sd < G::QL; ++sd)
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt)
      *reinterpret_cast<u32x4_t *>(qa + (sd * G::NT + nt) * G::THREADS * 16) = qf[nt][sd];
}

// A negative softmax scale is applied as a positive one on -q (exact), so the
// kernels only ever see c > 0.
__device__ __forceinline__ u32x4_t neg_bf16x8(u32x4_t x, uint32_t sign) {
  return u32x4_t{x[0] ^ sign, x[1] ^ sign, x[2] ^ sign, x[3] ^ sign};
}

// Q fragments of a prefill row tile: the tile's rows (rows tile_rows of a
// contiguous [., D] bf16 array starting at q) as one buffer range, so rows
// past the end read as zeros without a branch, and no wait on these loads
// comes before the first K/V tiles are requested.
template <class G>
__device__ __forceinline__ void load_q_rows(u32x4_t (&qf)[G::NT][G::SD], const __bf16 *q, int tile_rows, int rg,
                                            int lane, uint32_t qsign) {
  const auto rq = make_rsrc(q, (uint32_t)tile_rows * G::D * 2);
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const uint32_t lr = (uint32_t)((rg * G::NT + nt) * 32 + (lane & 31));
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd)
      qf[nt][sd] = neg_bf16x8(buf_load16(rq, (lr * G::D + 16 * sd + 8 * (lane >> 5)) * 2), qsign);
  }
}

template <class G>
__device__ __forceinline__ void qk_tile(f32x16_t (&s)[G::NT][G::KB], const u32x4_t (&qf)[G::NT][G::SD],
                                        const char *qa, const char *kt, int lane) {
  const char *base = kt + G::k_lane(lane);
  u32x4_t fb[G::NFQ];
#pragma unroll
  for (int f = 0; f < G::NFQ; ++f) fb[f] = *reinterpret_cast<const u32x4_t *>(base + G::k_frag(f % G::KB, f / G::KB));
#pragma unroll
  for (int f = 0; f < G::NFQ; ++f) {
    const int kb = f % G::KB, sd = f / G::KB;
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt)
      s[nt][kb] = mfma32(as_bf16x8(fb[f]), as_bf16x8(sd < G::QL ? q_lds<G>(qa, nt, sd) : qf[nt][sd]),
                         sd == 0 ? f32x16_t{} : s[nt][kb]);
  }
}

// Score masks of the kernels without an additive mask, applied to S of each
// tile (keys key0 ..) right after its QK^T.  Lane l holds keys
// key0 + kb*32 + (v/4)*8 + 4*(l/32) + v%4 of its row in s[nt][kb][v].
//
// TailMask removes keys >= n_keys (rare uniform branch: only the ragged last
// tile and padding tiles).
struct TailMask {
  int n_keys;
  template <class G>
  __device__ __forceinline__ void apply(f32x16_t (&s)[G::NT][G::KB], int key0, int lane) const {
    if (key0 + G::BN > n_keys) {
      const int h = lane >> 5;
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
  }
};

// CausalMask: the row of token t sees keys <= t.  The uniform branch is taken
// only by tiles that reach past the smallest token of the wave (the diagonal
// tiles, the ragged last tile and padding tiles; the source's n_keys is one
// past the largest token of the workgroup, so keys >= n_keys are removed too).
// The mask replaces scores, it does not add to them: a key after the token
// leaves no trace whatever its K holds.
template <int NT>
struct CausalMask {
  int t[NT];  // token of the lane's row in row block nt (huge for padding rows)
  int t_min;  // wave-uniform minimum of t
  template <class G>
  __device__ __forceinline__ void apply(f32x16_t (&s)[G::NT][G::KB], int key0, int lane) const {
    if (key0 + G::BN - 1 > t_min) {
      const int h = lane >> 5;
      int lim[G::NT];  // keys with offset > lim are after the token
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) lim[nt] = t[nt] - key0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = kb * 32 + (v >> 2) * 8 + (v & 3);
#pragma unroll
          for (int nt = 0; nt < G::NT; ++nt) s[nt][kb][v] = off > lim[nt] ? -INFINITY : s[nt][kb][v];
        }
    }
  }
};

// Empty asm statements are ordered side effects: pin_in redefines a value at
// a point (nothing that uses it can move above), pin_out consumes it (its
// computation cannot sink below).  Together with sched_barrier they hold a
// hand-interleaved MFMA / VALU sequence in place.
template <class T>
__device__ __forceinline__ void pin_in(T &x) {
  asm volatile("" : "+v"(x));
}
template <class T>
__device__ __forceinline__ void pin_out(const T &x) {
  asm volatile("" ::"v"(x));
}

// Softmax state carried from phase A into phase B of a tile step: the packed
// bf16 P words (w[nt][kb][i] holds keys 2i, 2i+1 of the lane's 16 in block kb),
// the running row sum and the reference max used for this tile's exponents.
template <class G>
struct PCarry {
  uint32_t w[G::NT][G::KB][8];
  float lsum[G::NT], m_use[G::NT];
};

// exp2 / bf16 pack / row sum of P pair i8 of block (nt, kb), with the
// reference max `mu` (a slot-local pinned copy).
template <class G, bool HAS_MASK>
__device__ __forceinline__ void p_pair(PCarry<G> &pc, const f32x16_t (&s)[G::NT][G::KB], int nt, int kb, int i8,
                                       float mu, float c) {  // mu: this slot's pinned reference max
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  const float x0 = s[nt][kb][2 * i8], x1 = s[nt][kb][2 * i8 + 1];
  const float e0 = HAS_MASK ? fast_exp2(x0 - mu) : fast_exp2(__builtin_fmaf(x0, c, -mu));
  const float e1 = HAS_MASK ? fast_exp2(x1 - mu) : fast_exp2(__builtin_fmaf(x1, c, -mu));
  pc.w[nt][kb][i8] = pack_bf16(e0, e1);
  pc.lsum[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pc.w[nt][kb][i8]), ones, pc.lsum[nt], false);
  pin_out(pc.w[nt][kb][i8]);
}

// P pairs [p0, p1) of one half (i8 < 4: the first 16 keys of each 32-key
// block, i8 >= 4: the second), numbered over (nt, kb, i8 % 4).
template <class G, bool HAS_MASK>
__device__ __forceinline__ void p_pairs(PCarry<G> &pc, const f32x16_t (&s)[G::NT][G::KB], int half, int p0, int p1,
                                        float c) {
  // re-pinning the reference max in place (no copy) keeps this slot's exps
  // from being hoisted into an earlier slot
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) pin_in(pc.m_use[nt]);
#pragma unroll
  for (int a = p0; a < p1; ++a) {
    const int nt = a / (G::KB * 4), kb = (a / 4) % G::KB, i8 = 4 * half + a % 4;
    p_pair<G, HAS_MASK>(pc, s, nt, kb, i8, pc.m_use[nt], c);
  }
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) pin_out(pc.lsum[nt]);
}

// u32x4 B fragment of P for (nt, kb, kk) from the packed words (bit-cast plain
// scalars, never ext-vector elements: hipcc folded a bit_cast of pb[..][i] to
// element 0 for every i)
template <class G>
__device__ __forceinline__ u32x4_t p_frag(const PCarry<G> &pc, int nt, int kb, int kk) {
  return u32x4_t{pc.w[nt][kb][4 * kk], pc.w[nt][kb][4 * kk + 1], pc.w[nt][kb][4 * kk + 2], pc.w[nt][kb][4 * kk + 3]};
}

// LAZYSUM: the rows whose half-tile sum went past 2^kTau (own lane or its
// partner) take the tile's max and move their reference when it exceeds the
// old one by more than kTau (the raw-unit threshold).  Returns per row
// whether it moved and the old reference (for the rescale); updates m, the
// exponents' reference and the threshold.
template <class G>
__device__ __forceinline__ bool lazy_redecide(WaveState<G> &ws, const f32x16_t (&s)[G::NT][G::KB],
                                              const bool (&trig)[G::NT], float c, bool (&grow)[G::NT],
                                              float (&m_old)[G::NT]) {
  bool any = false;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const bool row_trig = pair_max(trig[nt] ? 1.0f : 0.0f) > 0.0f;
    float mx = s[nt][0][0];
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = __builtin_fmaxf(mx, s[nt][kb][v]);
    mx = pair_max(mx);
    grow[nt] = row_trig && mx > ws.thr[nt];
    m_old[nt] = ws.m[nt];
    const float m_new = grow[nt] ? mx * c : ws.m[nt];
    ws.m[nt] = m_new;
    ws.mu[nt] = fmaxf(m_new, -kFloatMax);
    ws.thr[nt] = grow[nt] ? (m_new + kTau) * (1.0f / c) : ws.thr[nt];
    any |= grow[nt];
  }
  return __ballot(any) != 0;
}

// Phase A of one tile step: S(next) = K(next) Q^T on MFMA, interleaved with
// the online softmax of S (this tile) on the VALU.  c = softmax_scale*log2(e)
// > 0.  With a mask, mk (LDS) holds this tile's additive mask in log2 units,
// -inf for removed keys.  Computes the first half of P (the keys the first
// PV MFMAs consume), updates m, and returns whether any row's reference max
// moved: then O must be multiplied by alpha before PV.  la is alpha (1 for the
// rows that keep their reference), or with G::RARE_ALPHA its log2 (old
// reference - new, 0 for those rows): the caller takes the exp2 on that rare
// path, and rescales l there too.
//
// Slot f issues QK MFMA f and the K read GRP fragments ahead, and a slice of
// the softmax (before or after the MFMA, G::VFIRST): slot 0 the row max, slot
// 1 the cross-lane max, the rescale decision and la, later slots the exp2
// / bf16 pack / row sum of P pairs.
// sched_barrier(0) and the pins hold that order, so this wave's MFMAs run
// under its own VALU work; the second half of P is left to phase B, which
// balances the VALU load of the two phases.
//
// Lazy rescale: the reference max m of a row only moves when the row's tile
// max exceeds it by more than kTau, so p = 2^(s - m) <= 2^kTau and the O
// rescale (a VALU pass over every accumulator, skipped unless some row of the
// wave moved) is rare.  Exact: the final O/l uses one
// consistent reference per row.  The row sum is taken on the packed bf16 P
// (v_dot2_f32_bf16), so it normalises exactly the values multiplied into V;
// with G::RARE_ALPHA the tile's sum starts from zero (pc.lsum) and joins l at
// the end of phase B; otherwise it starts from l * alpha.
template <class G, bool HAS_MASK>
__device__ __forceinline__ bool phase_a(WaveState<G> &ws, PCarry<G> &pc, f32x16_t (&sn)[G::NT][G::KB],
                                        f32x16_t (&s)[G::NT][G::KB], float (&la)[G::NT],
                                        const u32x4_t (&qf)[G::NT][G::SD], const char *qa, const char *kt,
                                        const float *mk, float c, int lane) {
  constexpr int RA = G::GRP < G::NFQ ? G::GRP : G::NFQ;
  constexpr int NP = G::NT * G::KB * 4;  // P pairs of the first half
  constexpr int SLOTS = G::NFQ - 2;
  constexpr int PPS = (NP + SLOTS - 1) / SLOTS;
  // With at least one slot per pair, pairs are spaced evenly over slots
  // 2 .. NFQ-1 (one every SPA slots) so that no slot's VALU slice outgrows
  // its MFMA; otherwise PPS consecutive pairs per slot.
  constexpr int SPA = SLOTS >= NP && NP > 1 ? (SLOTS - 1) / (NP - 1) : 0;
  static_assert(SLOTS >= 1, "QK slots");
  // LAZYSUM: the first half's pairs over all NFQ slots, PPA per slot
  constexpr int PPA = (NP + G::NFQ - 1) / G::NFQ;
  static_assert(!G::LAZYSUM || (G::RARE_ALPHA && G::VFIRST && !HAS_MASK), "lazy sum: rare rescale, VALU first");
  if constexpr (G::LAZYSUM) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      pc.m_use[nt] = ws.mu[nt];
      pc.lsum[nt] = 0.0f;
    }
  }
  const int h = lane >> 5;
  const char *kbase = kt + G::k_lane(lane);

  u32x4_t fb[G::NFQ];
  u32x4_t ql[G::QL > 0 ? G::QL : 1][G::NT];
  f32x4_t m4[G::KB][4];
  float mx[G::NT];
  bool any = false;

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int sd = 0; sd < G::QL; ++sd)
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) ql[sd][nt] = q_lds<G>(qa, nt, sd);
#pragma unroll
  for (int f = 0; f < RA; ++f)
    fb[f] = *reinterpret_cast<const u32x4_t *>(kbase + G::k_frag(f % G::KB, f / G::KB));
  if constexpr (HAS_MASK) {
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) m4[kb][r4] = *reinterpret_cast<const f32x4_t *>(mk + kb * 32 + r4 * 8 + 4 * h);
  }
  __builtin_amdgcn_sched_barrier(0);

  auto qk_slot = [&](int f) {
    const int kb = f % G::KB, sd = f / G::KB;
    pin_in(fb[f]);
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      if (sd < G::QL) pin_in(ql[sd < G::QL ? sd : 0][nt]);
      sn[nt][kb] = mfma32(as_bf16x8(fb[f]), as_bf16x8(sd < G::QL ? ql[sd < G::QL ? sd : 0][nt] : qf[nt][sd]),
                          sd == 0 ? f32x16_t{} : sn[nt][kb]);
    }
    if (f + RA < G::NFQ) {
      const int g = f + RA;
      fb[g] = *reinterpret_cast<const u32x4_t *>(kbase + G::k_frag(g % G::KB, g / G::KB));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int f = 0; f < G::NFQ; ++f) {
    if (!G::VFIRST) qk_slot(f);
    if constexpr (G::LAZYSUM) {
      if (f * PPA < NP) p_pairs<G, HAS_MASK>(pc, s, 0, f * PPA, (f + 1) * PPA < NP ? (f + 1) * PPA : NP, c);
    } else if (f == 0) {
      // scores into log2 units (mask path) and the in-lane row max
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        if constexpr (HAS_MASK) {
#pragma unroll
          for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {  // removed keys stay -inf whatever their K holds
              const float mv = m4[kb][v / 4][v % 4];
              s[nt][kb][v] = mv == -INFINITY ? -INFINITY : __builtin_fmaf(s[nt][kb][v], c, mv);
            }
        }
        // one max3 per pair of scores; the pin keeps the chain (left free,
        // the compiler rebuilds it as a tree of max and max3 that takes 11
        // instructions for 16 scores instead of 8)
        float mloc = __builtin_fmaxf(s[nt][0][0], s[nt][0][1]);
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
          for (int v = kb == 0 ? 2 : 0; v < 16; v += 2) {
            mloc = __builtin_fmaxf(mloc, __builtin_fmaxf(s[nt][kb][v], s[nt][kb][v + 1]));
            pin_in(mloc);
          }
        mx[nt] = mloc;
        pin_out(mx[nt]);
      }
    } else if (f == 1) {
      bool grow = false, grow_row[G::NT];
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        const float m2 = pair_max(mx[nt]);
        if constexpr (G::RARE_ALPHA) {
          static_assert(!HAS_MASK, "raw-unit threshold: scores without an additive mask");
          mx[nt] = m2;  // raw units; scaled on the rare path
          grow_row[nt] = m2 > ws.thr[nt];
        } else {
          mx[nt] = HAS_MASK ? m2 : m2 * c;  // -inf * c = -inf (c > 0)
          grow_row[nt] = mx[nt] > ws.m[nt] + kTau;
        }
        grow |= grow_row[nt];
      }
      any = __ballot(grow) != 0;
      // per row: a row's reference moves only on its own scores, so its
      // result never depends on the other rows of the wave (alpha = 1 leaves
      // the rows that keep theirs bit-identical).  A growing row's tile max
      // exceeds its old reference, so it is the new one, and is finite:
      // exp2(m - mx) is 0 for a first live tile (m = -inf).  A row with no
      // live key yet keeps m = -inf; its exponents use the lowest float
      // instead (-kFloatMax), which gives p = 0 for its -inf scores without a NaN.
      if constexpr (G::RARE_ALPHA) {
        if (any) {  // rare: the rows whose reference moves
#pragma unroll
          for (int nt = 0; nt < G::NT; ++nt) {
            const float mxc = mx[nt] * c;
            const float m_new = grow_row[nt] ? mxc : ws.m[nt];
            la[nt] = grow_row[nt] ? ws.m[nt] - mxc : 0.0f;
            ws.m[nt] = m_new;
            ws.mu[nt] = fmaxf(m_new, -kFloatMax);
            ws.thr[nt] = grow_row[nt] ? (m_new + kTau) * (1.0f / c) : ws.thr[nt];
          }
        }
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          pc.m_use[nt] = ws.mu[nt];
          pc.lsum[nt] = 0.0f;
          pin_out(pc.m_use[nt]);
          pin_out(pc.lsum[nt]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          const float m_new = grow_row[nt] ? mx[nt] : ws.m[nt];
          la[nt] = grow_row[nt] ? fast_exp2(ws.m[nt] - mx[nt]) : 1.0f;
          ws.m[nt] = m_new;
          pc.m_use[nt] = fmaxf(m_new, -kFloatMax);
          pc.lsum[nt] = ws.l[nt] * la[nt];
          pin_out(pc.m_use[nt]);
          pin_out(pc.lsum[nt]);
          pin_out(la[nt]);
        }
      }
    } else if constexpr (SPA > 0) {
      if ((f - 2) % SPA == 0 && (f - 2) / SPA < NP) p_pairs<G, HAS_MASK>(pc, s, 0, (f - 2) / SPA, (f - 2) / SPA + 1, c);
    } else {
      const int p0 = (f - 2) * PPS, p1 = (f - 1) * PPS < NP ? (f - 1) * PPS : NP;
      if (p0 < p1) p_pairs<G, HAS_MASK>(pc, s, 0, p0, p1, c);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (G::VFIRST) qk_slot(f);
  }
  if constexpr (G::LAZYSUM) {
    bool trig[G::NT], t = false;
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      trig[nt] = pc.lsum[nt] > kSumTrig;
      t |= trig[nt];
    }
    if (__ballot(t) != 0) {  // rare
      bool grow[G::NT];
      float m_old[G::NT];
      any = lazy_redecide<G>(ws, s, trig, c, grow, m_old);
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        la[nt] = grow[nt] ? m_old[nt] - ws.m[nt] : 0.0f;
        pc.m_use[nt] = ws.mu[nt];
        pc.lsum[nt] = 0.0f;
      }
      p_pairs<G, HAS_MASK>(pc, s, 0, 0, NP, c);  // the first half again (same bits where the reference held)
    }
  }
  return any;
}

// Phase B: O^T += V^T P^T for one tile.  Slots before MT compute the second
// half of P (needed from PV MFMA MT on), later ones the staging work of the
// tile step (`work(k)`, k = 0, 1, 2).  The A fragment (d rows mt*32 + lane%32,
// k-slots j = 0..7 of lane-half h) must hold the keys P's B fragment holds:
// kb*32 + 16kk + 8(j/4) + 4h + j%4.  Two transposing reads (t = j/4) fetch
// it: in 16-lane group g the reading lane 4m + j names the 8 bytes
// V[kb*32 + 16kk + 8t + 4h + j][mt*32 + 16(g%2) + 4m ..], and output lane
// 16g + 4m + c receives element c of those four rows.  Row bases are
// multiples of 4, so v_row(base + j) = v_row(base) + v_row(j).  Over tile
// images (G::DMA) V^T already holds those keys in that order: one 16-byte
// read at vt_off.
// PV A fragment q of a directly copied V tile (G::EDMA): the same rows and
// columns as the staged read above, at their row-major, half-swapped place:
// logical 16-byte chunk c of row r sits at r*128 + 16*(c ^ 4*((r >> 1) & 1)).
// The row offsets of the fragments (8t + 16kk + 32kb) keep bit 1, so the swap
// is fixed per lane.  In each half-wave the four rows j = 0..3 then fall in
// four different quarters of the 64 banks.
template <class G>
__device__ __forceinline__ u32x4_t v_frag_edma(const char *vt, int lane, int q) {
  const int h = lane >> 5, j = (lane >> 2) & 3, m = lane & 3, g2 = (lane >> 4) & 1;
  const int mt = q % G::MT, kk = (q / G::MT) % 2, kb = q / (2 * G::MT);
  const char *p = vt + (4 * h + j) * 128 + ((mt ^ ((j >> 1) & 1)) << 6) + (2 * g2 + (m >> 1)) * 16 + (m & 1) * 8 +
                  (kb * 32 + kk * 16) * 128;
  const u32x2_t a0 = lds_read_tr16(p), a1 = lds_read_tr16(p + 8 * 128);
  return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
}

template <class G, bool HAS_MASK, class Work>
__device__ __forceinline__ void phase_b(WaveState<G> &ws, PCarry<G> &pc, const f32x16_t (&s)[G::NT][G::KB],
                                        float c, const char *vt, int lane, Work &&work) {
  constexpr int RA = G::GRP < G::NFV ? G::GRP : G::NFV;
  constexpr int NP = G::NT * G::KB * 4;                 // P pairs of the second half
  constexpr int PPS = (NP + G::MT - 1) / G::MT;          // spread over the first MT slots
  constexpr int PSLOTS = (NP + PPS - 1) / PPS;
  // With MT >= NP: one pair every SPB slots of the first MT, the three
  // staging items every WS slots from slot MT on (even VALU per slot).
  constexpr int SPB = G::MT >= NP ? G::MT / NP : 0;
  constexpr int WS = (G::NFV - 1 - G::MT) / 2;
  static_assert(SPB == 0 || (WS >= 1 && G::MT + 2 * WS < G::NFV), "phase B schedule");
  const int h = lane >> 5, j = (lane >> 2) & 3, m = lane & 3, g2 = (lane >> 4) & 1;
  const char *vbase = vt + (G::DMA ? 0 : G::v_row(4 * h) + G::v_row(j) + 32 * g2 + 8 * m);
  // V^T (DMA): d = mt*32 + lane%32, and the swizzle sees d bits 2, 3 only
  const int vto = G::vt_off(lane & 31, 0, h);
  u32x4_t fb[G::NFV];
  auto read = [&](int q) {
    const int mt = q % G::MT, kk = (q / G::MT) % 2, kb = q / (2 * G::MT);
    if constexpr (G::DMA) {
      fb[q] = *reinterpret_cast<const u32x4_t *>(vt + vto + G::vt_off(32 * mt, kk, 0));
    } else if constexpr (G::EDMA) {
      fb[q] = v_frag_edma<G>(vt, lane, q);
    } else {
      const char *p = vbase + G::v_row(kb * 32 + kk * 16) + 64 * mt;
      const u32x2_t a0 = lds_read_tr16(p), a1 = lds_read_tr16(p + G::v_row(8));
      fb[q] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    }
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < RA; ++q) read(q);
  __builtin_amdgcn_sched_barrier(0);
  static_assert(!G::LAZYSUM || PSLOTS <= G::MT, "lazy sum: the second half is complete before its MFMAs");
  auto pv_slot = [&](int q) {
    const int mt = q % G::MT, kk = (q / G::MT) % 2, kb = q / (2 * G::MT);
    pin_in(fb[q]);
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      if constexpr (G::PVPRIO) __builtin_amdgcn_s_setprio(1);
      ws.o[nt][mt] = mfma32(as_bf16x8(fb[q]), as_bf16x8(p_frag(pc, nt, kb, kk)), ws.o[nt][mt]);
      if constexpr (G::PVPRIO) __builtin_amdgcn_s_setprio(0);
    }
    if (q + RA < G::NFV) read(q + RA);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int q = 0; q < G::NFV; ++q) {
    if (!G::VFIRST) pv_slot(q);
    if constexpr (G::LAZYSUM) {
      if (q == G::MT) {  // the second half, before the first MFMA that uses it
        bool trig[G::NT], t = false;
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          trig[nt] = pc.lsum[nt] > kSumTrig;  // both halves so far: conservative
          t |= trig[nt];
        }
        if (__ballot(t) != 0) {  // rare: O already holds the first half's products
          bool grow[G::NT];
          float m_old[G::NT];
          lazy_redecide<G>(ws, s, trig, c, grow, m_old);
          const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
          for (int nt = 0; nt < G::NT; ++nt) {
            const float alpha = grow[nt] ? fast_exp2(m_old[nt] - ws.m[nt]) : 1.0f;
            ws.l[nt] *= alpha;
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] *= alpha;
            float t1 = 0.0f;  // the first half's sum, in phase A's order
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
              for (int i8 = 0; i8 < 4; ++i8)
                t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pc.w[nt][kb][i8]), ones, t1, false);
            pc.lsum[nt] = t1 * alpha;
            pc.m_use[nt] = ws.mu[nt];
          }
          p_pairs<G, HAS_MASK>(pc, s, 1, 0, NP, c);  // the second half again
        }
      }
    }
    if constexpr (SPB > 0) {
      if (q % SPB == 0 && q / SPB < NP) p_pairs<G, HAS_MASK>(pc, s, 1, q / SPB, q / SPB + 1, c);
      else if (q >= G::MT && (q - G::MT) % WS == 0 && (q - G::MT) / WS <= 2) work((q - G::MT) / WS);
    } else if (q < PSLOTS) {
      p_pairs<G, HAS_MASK>(pc, s, 1, q * PPS, (q + 1) * PPS < NP ? (q + 1) * PPS : NP, c);
    } else {
      const int k = q - PSLOTS;
      if (k <= 2) work(k);
      if (q == G::NFV - 1)  // fewer slots than work items: the rest goes here
        for (int r = k + 1; r <= 2; ++r) work(r);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (G::VFIRST) pv_slot(q);
  }
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) ws.l[nt] = G::RARE_ALPHA ? ws.l[nt] + pc.lsum[nt] : pc.lsum[nt];
}

// ------------------------------------------------------------------ core loop

// The pipelined key loop of all three kernels.  LDS holds two K buffers and
// two V buffers; iteration `it` (every split's tile `it`) reads K(it+1) and
// V(it), writes K(it+2) into the K buffer K(it) used and V(it+1) into the
// other V buffer, and issues the global loads of K(it+3) and V(it+2) into the
// register stage.  Tiles past the last one read as zeros and are fully
// masked (p = 0), including the padding step of an odd iteration count.
// Without an additive mask, `mk` masks the scores of each tile (TailMask,
// CausalMask).  `fresh` starts a new softmax state; otherwise the loop
// continues the one in `ws` (same log2 units: c must give true scores times
// log2(e)).  `tid` is threadIdx.x.  Returns with the LDS free (barrier
// passed).
template <class G, bool HAS_MASK, class Src, class Mask>
__device__ __forceinline__ void flash_loop(WaveState<G> &ws, const Src &src, const u32x4_t (&qf)[G::NT][G::SD],
                                           char *smem, float c, const Mask &mk, bool fresh, unsigned tid) {
  static_assert(!G::RARE_ALPHA, "the rare-path rescale state is set up by flash_loop_dma");
  const int lane = tid & 63;
  const int sp = __builtin_amdgcn_readfirstlane((int)(tid >> 6)) / G::RG;
  const int n_tiles = (src.n_keys + G::BN - 1) / G::BN;
  const int n_iter = (n_tiles + G::NSPLIT - 1) / G::NSPLIT;
  if (fresh) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      ws.m[nt] = -INFINITY;
      ws.l[nt] = 0.0f;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] = f32x16_t{};
    }
  }
  if (n_iter <= 0) return;

  char *const kbuf = smem, *const vbuf = smem + 2 * G::KSLOT;
  const char *const qa = smem + G::QOFF + tid * 16;  // this thread's LDS Q slots (G::QL > 0)
  // Prologue: K(0), V(0) and K(1) in one round trip (a second register stage
  // that is only live here), then K(2), V(1) in flight.
  typename Src::Stage st, st1;
  const int64_t b0 = src.tile_base(0), b1 = src.tile_base(1);
  src.load_k(st, 0, b0, tid);
  src.load_v(st, 0, b0, tid);
  src.load_k(st1, 1, b1, tid);
  q_to_lds<G>(qf, smem + G::QOFF + tid * 16);  // own Q slots: after the tile loads are on their way
  src.store_k(st, kbuf, tid);
  src.store_v(st, vbuf, 0, tid);
  src.store_k(st1, kbuf + G::KSLOT, tid);
  int64_t bv = src.tile_base(2);  // V(it+2) base
  src.load_k(st, 2, bv, tid);
  src.load_v(st, 1, b1, tid);
  int64_t bk = src.tile_base(3);  // K(it+3) base
  __syncthreads();

  f32x16_t s[G::NT][G::KB];
  qk_tile<G>(s, qf, qa, kbuf + sp * G::KTILE, lane);
  if constexpr (!HAS_MASK) mk.template apply<G>(s, sp * G::BN, lane);
  // iteration 0 writes K(2) into K(0)'s buffer: every wave must have read
  // K(0) first
  __syncthreads();

  // One tile step: S holds S(it) on entry, SN receives S(it+1).  The loop
  // below alternates the two register sets instead of copying S each step;
  // an odd iteration count is padded with one all-masked zero tile.
  auto step = [&](int it, f32x16_t (&S)[G::NT][G::KB], f32x16_t (&SN)[G::NT][G::KB]) {
    const int cur = it & 1;
    char *const kcur = kbuf + cur * G::KSLOT, *const knext = kbuf + (cur ^ 1) * G::KSLOT;
    char *const vcur = vbuf + cur * G::VSLOT, *const vnext = vbuf + (cur ^ 1) * G::VSLOT;

    PCarry<G> pc;
    float la[G::NT];
    const bool any =
        phase_a<G, HAS_MASK>(ws, pc, SN, S, la, qf, qa, knext + sp * G::KTILE,
                             reinterpret_cast<const float *>(vcur + G::NSPLIT * G::VTILE) + sp * G::BN, c, lane);
    if (any) {  // rare: the rows whose reference moved rescale O (and l) (alpha = 1 for the others)
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        const float alpha = G::RARE_ALPHA ? fast_exp2(la[nt]) : la[nt];
        if constexpr (G::RARE_ALPHA) ws.l[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] *= alpha;
      }
    }

    // PV(it); stage K(it+2) and V(it+1); issue K(it+3) and V(it+2)
    phase_b<G, HAS_MASK>(ws, pc, S, c, vcur + sp * G::VTILE, lane, [&](int k) {
      if (k == 0) src.store_k(st, kcur, tid);
      if (k == 1) src.store_v(st, vnext, it + 1, tid);
      if (k == 2) {
        src.load_k(st, it + 3, bk, tid);
        src.load_v(st, it + 2, bv, tid);
        bv = bk;
        bk = src.tile_base(it + 4);
      }
    });
    __syncthreads();

    if constexpr (!HAS_MASK) mk.template apply<G>(SN, ((it + 1) * G::NSPLIT + sp) * G::BN, lane);
  };

  f32x16_t s2[G::NT][G::KB];
  const int n_even = (n_iter + 1) & ~1;
  for (int it = 0; it < n_even; it += 2) {
    step(it, s, s2);
    step(it + 1, s2, s);
  }
}

// The key loop over tiles copied by direct loads: tile images (G::DMA, one
// key split) or the encoder's own rows (G::EDMA, each wave reading its key
// split's tile of every buffer).  Three K buffers
// (kA, kB, kC) and three V buffers: at step `it` they hold K(it), K(it+1),
// K(it+2) and V(it), V(it+1), V(it+2) in an order that rotates with it % 3.
// Phase A reads K(it+1), phase B reads V(it), and the step copies K(it+3)
// into K(it)'s buffer and V(it+2) into V(it-1)'s, both released by the
// barrier that ended the step before.  Before its closing barrier a step
// waits for the copies of the step before (K(it+2), V(it+1), which the next
// step reads) and leaves its own in flight, so every copy has a full step
// to land.  The buffers are __restrict__ parameters and every step names
// its four by role (the loop runs six steps per pass: three rotations times
// the S / SN alternation), so the compiler can tell that a copy in flight
// never aliases the LDS reads that follow it; otherwise it would wait for
// every copy before each LDS read.  Same phases, schedule and masks as
// flash_loop.
template <class G, class Src, class Mask>
__device__ __forceinline__ void dma_loop_body(WaveState<G> &ws, const Src &src,
                                              const u32x4_t (&qf)[G::NT][G::SD], char *__restrict__ kA,
                                              char *__restrict__ kB, char *__restrict__ kC, char *__restrict__ vA,
                                              char *__restrict__ vB, char *__restrict__ vC,
                                              char *__restrict__ qa, float c, const Mask &mk, int lane,
                                              int wave, int n_iter) {
  src.copy_k(kA, 0, wave, lane);
  src.copy_v(vA, 0, wave, lane);
  src.copy_k(kB, 1, wave, lane);
  src.copy_v(vB, 1, wave, lane);
  src.copy_k(kC, 2, wave, lane);
  q_to_lds<G>(qf, qa);  // own Q slots: after the tile copies are on their way
  // K(0), V(0) and K(1) are read before the first step's copies are waited
  // for; V(1) and K(2), the last two issued, may still be in flight
  Src::wait_step(wave);
  lds_barrier();

  // key split of this wave (its tile of each iteration: sp * KTILE, sp * VTILE)
  const int sp = G::NSPLIT > 1 ? wave / G::RG : 0;
  f32x16_t s[G::NT][G::KB], s2[G::NT][G::KB];
  qk_tile<G>(s, qf, qa, kA + sp * G::KTILE, lane);
  mk.template apply<G>(s, sp * G::BN, lane);
  if constexpr (G::LAZYSUM) {
    // a row without a reference takes the first tile's max as its own, so
    // the first step does not have to leave the common path to set it
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      float mx = s[nt][0][0];
#pragma unroll
      for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = __builtin_fmaxf(mx, s[nt][kb][v]);
      mx = pair_max(mx);
      if (ws.m[nt] == -INFINITY && mx > -INFINITY) {
        ws.m[nt] = mx * c;
        ws.mu[nt] = ws.m[nt];
        ws.thr[nt] = (ws.m[nt] + kTau) * (1.0f / c);
      }
    }
  }
  lds_barrier();  // K(0) read by every wave before K(3) replaces it

  // kr: K(it+1), read; kw: K(it)'s buffer, receives K(it+3); vr: V(it), read;
  // vw: V(it-1)'s buffer, receives V(it+2)
  auto step = [&](int it, char *__restrict__ kr, char *__restrict__ kw, char *__restrict__ vr,
                  char *__restrict__ vw, f32x16_t (&S)[G::NT][G::KB], f32x16_t (&SN)[G::NT][G::KB]) {
    PCarry<G> pc;
    float la[G::NT];
    const bool any = phase_a<G, false>(ws, pc, SN, S, la, qf, qa, kr + sp * G::KTILE, nullptr, c, lane);
    if (any) {  // rare: the rows whose reference moved rescale O (and l) (alpha = 1 for the others)
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        const float alpha = G::RARE_ALPHA ? fast_exp2(la[nt]) : la[nt];
        if constexpr (G::RARE_ALPHA) ws.l[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] *= alpha;
      }
    }
    phase_b<G, false>(ws, pc, S, c, vr + sp * G::VTILE, lane, [&](int k) {
      if (k == 0) src.copy_k(kw, it + 3, wave, lane);
      if (k == 1) src.copy_v(vw, it + 2, wave, lane);
    });
    Src::wait_step(wave);  // the step before's copies have landed
    lds_barrier();
    mk.template apply<G>(SN, ((it + 1) * G::NSPLIT + sp) * G::BN, lane);
  };
  for (int it = 0; it < n_iter; it += 6) {
    step(it, kB, kA, vA, vC, s, s2);
    if (it + 1 >= n_iter) break;
    step(it + 1, kC, kB, vB, vA, s2, s);
    if (it + 2 >= n_iter) break;
    step(it + 2, kA, kC, vC, vB, s, s2);
    if (it + 3 >= n_iter) break;
    step(it + 3, kB, kA, vA, vC, s2, s);
    if (it + 4 >= n_iter) break;
    step(it + 4, kC, kB, vB, vA, s, s2);
    if (it + 5 >= n_iter) break;
    step(it + 5, kA, kC, vC, vB, s2, s);
  }
  wait_vm<0>();  // no copy may still be writing into LDS the epilogue reuses
  lds_barrier();
}

template <class G, class Src, class Mask>
__device__ __forceinline__ void flash_loop_dma(WaveState<G> &ws, const Src &src,
                                               const u32x4_t (&qf)[G::NT][G::SD], char *smem, float c, const Mask &mk,
                                               bool fresh, unsigned tid) {
  static_assert(G::LINEAR && (G::EDMA || G::NSPLIT == 1), "tile images: one key split");
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int n_iter = ((src.n_keys + G::BN - 1) / G::BN + G::NSPLIT - 1) / G::NSPLIT;
  if (fresh) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      ws.m[nt] = -INFINITY;
      ws.l[nt] = 0.0f;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) ws.o[nt][mt] = f32x16_t{};
    }
  }
  if constexpr (G::RARE_ALPHA) {  // from m (fresh: -inf, so any live key moves it)
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      ws.mu[nt] = fmaxf(ws.m[nt], -kFloatMax);
      ws.thr[nt] = ws.m[nt] == -INFINITY ? -INFINITY : (ws.m[nt] + kTau) * (1.0f / c);
    }
  }
  if (n_iter <= 0) {  // no key: copies issued before the loop (the encoder's residual rows) land first
    wait_vm<0>();
    return;
  }
  char *const vbuf = smem + 3 * G::KSLOT;
  dma_loop_body<G>(ws, src, qf, smem, smem + G::KSLOT, smem + 2 * G::KSLOT, vbuf, vbuf + G::VSLOT,
                   vbuf + 2 * G::VSLOT, smem + G::QOFF + tid * 16, c, mk, lane, wave, n_iter);
}

// Merge the NSPLIT key-split partial states into the split-0 waves (LDS).
template <class G>
__device__ __forceinline__ void merge_splits(WaveState<G> &ws, char *smem) {
  if constexpr (G::NSPLIT > 1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % G::RG, sp = wave / G::RG;
    constexpr int NREG = G::NT * (G::MT * 16 + 2);
    float *red = reinterpret_cast<float *>(smem);
    static_assert((G::NSPLIT - 1) * G::RG * NREG * 64 * 4 <= G::LDS, "merge space");  // G::MERGE
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

// ------------------------------------------------------------------ encoder kernel

template <class G, bool F32IN, bool HAS_MASK, int ROPE>
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
  // (fragment sd holds d = 16 sd + 8 hh ..; both RoPE pairings stay inside a
  // lane: interleaved pairs inside a fragment, rotate-half pairs fragment sd
  // with sd + SD/2)
  u32x4_t qf[G::NT][G::SD];
  const char *qb = reinterpret_cast<const char *>(a.q) + (b * a.qs[0] + h * a.qs[1]) * ES;
  // This tile's rows as one buffer range ending with the last row's data
  // (row stride < 2^24 bytes, checked on the host, so offsets fit 32 bits):
  // rows past Sq read as zeros without a branch.
  const uint32_t qrow = (uint32_t)(a.qs[2] * ES);
  const int row0 = qt * G::BM, nrow = min(a.Sq - row0, G::BM);
  const auto rq = make_rsrc(qb + (int64_t)row0 * a.qs[2] * ES, (uint32_t)(nrow - 1) * qrow + G::D * ES);
  // bf16 rows without a rotation are the fragments as loaded: no VALU work
  // touches them before the first MFMA, so no wait on these loads comes
  // before the tile copies are issued (the sign of q, for a negative scale,
  // is applied on a branch of its own).  fp32 rows are rounded and rotated
  // rows rotated here, which waits for them.
  constexpr bool RAW = !F32IN && ROPE == 0;
#pragma unroll
  for (int nt = 0; nt < G::NT && RAW; ++nt)
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd)
      qf[nt][sd] = buf_load16(rq, (uint32_t)((rg * G::NT + nt) * 32 + l32) * qrow + (16 * sd + 8 * hh) * ES);
  if (RAW && a.q_neg) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
      for (int sd = 0; sd < G::SD; ++sd) qf[nt][sd] = neg_bf16x8(qf[nt][sd], qsign);
  }
#pragma unroll
  for (int nt = 0; nt < G::NT && !RAW; ++nt) {
    const int lrow = (rg * G::NT + nt) * 32 + l32, row = row0 + lrow;
    float f[G::SD][8];
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd) {
      const uint32_t off = (uint32_t)lrow * qrow + (16 * sd + 8 * hh) * ES;
      u32x4_t x[F32IN ? 2 : 1];
      x[0] = buf_load16(rq, off);
      if constexpr (F32IN) x[1] = buf_load16(rq, off + 16);
      unpack8<F32IN>(x, f[sd]);
    }
    if (ROPE != 0 && row < a.Sq) {
      const float *rc = a.rope_cos + b * a.rope_sb + (int64_t)row * (G::D / 2);
      const float *rs = a.rope_sin + b * a.rope_sb + (int64_t)row * (G::D / 2);
      if constexpr (ROPE == 1) {
#pragma unroll
        for (int sd = 0; sd < G::SD / 2; ++sd) {
          const int k0 = 16 * sd + 8 * hh;
          const f32x4_t c0 = ldg<f32x4_t>(rc + k0), c1 = ldg<f32x4_t>(rc + k0 + 4);
          const f32x4_t s0 = ldg<f32x4_t>(rs + k0), s1 = ldg<f32x4_t>(rs + k0 + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            rot_pair(f[sd][e], f[sd + G::SD / 2][e], e < 4 ? c0[e] : c1[e - 4], e < 4 ? s0[e] : s1[e - 4]);
        }
      } else if constexpr (ROPE == 2) {
#pragma unroll
        for (int sd = 0; sd < G::SD; ++sd) {
          const int k0 = 8 * sd + 4 * hh;
          const f32x4_t c = ldg<f32x4_t>(rc + k0), sn = ldg<f32x4_t>(rs + k0);
#pragma unroll
          for (int i = 0; i < 4; ++i) rot_pair(f[sd][2 * i], f[sd][2 * i + 1], c[i], sn[i]);
        }
      }
    }
#pragma unroll
    for (int sd = 0; sd < G::SD; ++sd) qf[nt][sd] = neg_bf16x8(pack8(f[sd]), qsign);
  }

  // keys of this batch row: all S_kv, or its right-padded length
  const int n_keys =
      a.key_len ? __builtin_amdgcn_readfirstlane(min(max(a.key_len[b], 0), a.Skv)) : a.Skv;
  EncSrc<G, F32IN, HAS_MASK> src;
  src.kb = reinterpret_cast<const char *>(a.k) + (b * a.ks[0] + h * a.ks[1]) * ES;
  src.vb = reinterpret_cast<const char *>(a.v) + (b * a.vs[0] + h * a.vs[1]) * ES;
  src.krow = (uint32_t)(a.ks[2] * ES);
  src.vrow = (uint32_t)(a.vs[2] * ES);
  src.kstep = (int64_t)G::NSPLIT * G::BN * a.ks[2] * ES;
  src.vstep = (int64_t)G::NSPLIT * G::BN * a.vs[2] * ES;
  src.n_keys = n_keys;
  src.mask = HAS_MASK ? a.mask + b * a.mask_sb : nullptr;

  WaveState<G> ws;
  if constexpr (G::EDMA) {
    static_assert(!F32IN && !HAS_MASK, "direct copies: bf16 rows, no additive mask");
    // the residual rows land with the first tiles: the loop's first wait covers them (with no key
    // the loop does not run and waits for them itself)
    if (a.res_out)
      ResRows<G>::copy(a.res + ((int64_t)b * a.Sq + row0) * (a.H * G::D) + h * G::D, nrow, a.H * G::D,
                  smem + G::LDS - G::RES, __builtin_amdgcn_readfirstlane(wave), lane);
    EncDmaSrc<G> ds;
    ds.kb = src.kb;
    ds.vb = src.vb;
    ds.krow = src.krow;
    ds.vrow = src.vrow;
    ds.kstep = src.kstep;
    ds.vstep = src.vstep;
    ds.n_keys = n_keys;
    ds.init(__builtin_amdgcn_readfirstlane(wave), lane);
    flash_loop_dma<G>(ws, ds, qf, smem, a.c, TailMask{n_keys}, true, threadIdx.x);
  } else {
    flash_loop<G, HAS_MASK>(ws, src, qf, smem, a.c, TailMask{n_keys}, true, threadIdx.x);
  }

  // The residual rows are read before the split merge, so their latency
  // overlaps it.
  const int HD = a.H * G::D;
  f32x4_t resv[G::NT][G::MT][4];
  if (!G::EDMA && a.res_out && sp == 0) {
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      const int row = qt * G::BM + (rg * G::NT + nt) * 32 + l32;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int64_t off = ((int64_t)b * a.Sq + row) * HD + h * G::D + mt * 32 + r4 * 8 + 4 * hh;
          resv[nt][mt][r4] = row < a.Sq ? ldg<f32x4_t>(a.res + off) : f32x4_t{0, 0, 0, 0};
        }
    }
  }
  merge_splits<G>(ws, smem);
  if (sp != 0) return;
  if (G::EDMA && a.res_out) {  // residual rows from LDS (ResRows; merge_splits uses other bytes)
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          resv[nt][mt][r4] = ResRows<G>::read(smem + G::LDS - G::RES, (rg * G::NT + nt) * 32 + l32, mt * 32 + r4 * 8 + 4 * hh);
  }

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
          if constexpr (G::EDMA) {  // back into the row's LDS copy; stored by whole rows below
            const int lr = (rg * G::NT + nt) * 32 + l32;
            *reinterpret_cast<f32x4_t *>(smem + G::LDS - G::RES + ResRows<G>::offset(lr, d0)) = resv[nt][mt][r4] + val;
          } else {
            const int64_t off = ((int64_t)b * a.Sq + row) * HD + h * G::D + d0;
            *reinterpret_cast<f32x4_t *>(a.res_out + off) = resv[nt][mt][r4] + val;
          }
        }
      }
  }
  if constexpr (G::EDMA) {
    if (a.res_out) {
      // this wave's rows of residual_out, four whole 256-byte rows per store
      // (a lane per 16 bytes) instead of 32-byte pieces of 32 rows, and
      // non-temporal: measured 1-3% faster per block than either alone
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes above are done
      __builtin_amdgcn_wave_barrier();
      const char *rl = smem + G::LDS - G::RES;
#pragma unroll
      for (int i = 0; i < G::NT * 32 / 4; ++i) {
        const int r = rg * G::NT * 32 + 4 * i + (lane >> 4), c = lane & 15, row = qt * G::BM + r;
        if (row < a.Sq)
          __builtin_nontemporal_store(
              *reinterpret_cast<const f32x4_t *>(rl + ResRows<G>::offset(r, 4 * c)),
              reinterpret_cast<f32x4_t *>(a.res_out + ((int64_t)b * a.Sq + row) * HD + h * G::D + 4 * c));
      }
    }
  }
}

// ------------------------------------------------------------------ prefill kernel

// O * o_scale / l and the lse for the rows of one prefill row tile: to the
// bf16 output and the caller's lse, or (HANDOFF) in fp32 to the handoff
// buffers [Hkv*rows, D] and [Hkv*rows], from where the current-token kernel
// continues the softmax.  Both forms share every instruction but the store,
// which keeps the register allocation of the key loop ahead of them alike.
template <class G, bool HANDOFF>
__device__ __forceinline__ void prefill_epilogue(const WaveState<G> &ws, const PrefillLaunch &a, int rt, int kvh,
                                                 int rg, int lane, float o_scale) {
  const int rows = a.G * a.Lq;
  const int64_t row_base = (int64_t)kvh * rows;
  const int l32 = lane & 31, hh = lane >> 5;
  float *const lse = HANDOFF ? a.ws_ml : a.lse;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int r = rt * G::BM + (rg * G::NT + nt) * 32 + l32;
    const float lt = pair_sum(ws.l[nt]);
    if (r >= rows) continue;
    const float inv = lt > 0.0f ? o_scale / lt : 0.0f;
    if (lse && hh == 0) lse[row_base + r] = lt > 0.0f ? (ws.m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = mt * 32 + r4 * 8 + 4 * hh;
        const float o0 = ws.o[nt][mt][4 * r4 + 0] * inv, o1 = ws.o[nt][mt][4 * r4 + 1] * inv;
        const float o2 = ws.o[nt][mt][4 * r4 + 2] * inv, o3 = ws.o[nt][mt][4 * r4 + 3] * inv;
        if constexpr (HANDOFF)
          *reinterpret_cast<f32x4_t *>(a.ws_o + (row_base + r) * G::D + d0) = f32x4_t{o0, o1, o2, o3};
        else
          *reinterpret_cast<u32x2_t *>(a.out + (row_base + r) * G::D + d0) =
              u32x2_t{pack_bf16(o0, o1), pack_bf16(o2, o3)};
      }
  }
}

template <class G, bool HANDOFF>
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
  load_q_rows<G>(qf, a.q + (row_base + rt * G::BM) * G::D, min(rows - rt * G::BM, G::BM), rg, lane, qsign);

  WaveState<G> ws;
  if constexpr (G::DMA) {
    TileImgSrc<G> src;
    src.img = a.img + (int64_t)kvh * a.n_tiles * TileImgSrc<G>::TIMG;
    src.n_tiles = a.n_tiles;
    src.n_keys = a.L_act;
    flash_loop_dma<G>(ws, src, qf, smem, a.c, TailMask{a.L_act}, true, threadIdx.x);
  } else {
    PagedSrc<G> src;
    src.kc = a.kc;
    src.vc = a.vc;
    src.bt = (const __attribute__((address_space(4))) int32_t *)(a.bt);
    src.head_off = (int64_t)kvh * a.bs * G::D;
    src.blk_stride = (int64_t)a.Hkv * a.bs * G::D;
    src.bs = a.bs;
    src.n_keys = a.L_act;
    flash_loop<G, false>(ws, src, qf, smem, a.c, TailMask{a.L_act}, true, threadIdx.x);
  }

  prefill_epilogue<G, HANDOFF>(ws, a, rt, kvh, rg, lane, a.v_scale);
}

// Causal attention among the current tokens (bf16 K/V [Hkv, Lq, D]): the row
// of token t sees current keys 0..t.  With a history the online softmax
// continues the history kernel's handed-off state (the log-sum-exp merge of
// the two parts, exact: the state passes in fp32); without one it starts
// fresh.  A row tile's last token bounds the keys it reads, so the tiles of
// the latest token blocks carry the most work and are dispatched first.
template <class G>
__global__ __launch_bounds__(G::THREADS) __attribute__((amdgpu_waves_per_eu(G::WPE, G::WPE)))
void prefill_current_kernel(PrefillLaunch a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];  // G::LDS bytes
  const int rows = a.G * a.Lq;
  const int n_rt = (rows + G::BM - 1) / G::BM;
  const int total = n_rt * a.Hkv, i = blockIdx.x;
  int rt, kvh;
  if (a.Lq % G::BM == 0) {  // whole row tiles per head: latest token block first
    const int nb = a.Lq / G::BM, per = a.G * a.Hkv;
    const int tb = nb - 1 - i / per, g = (i % per) / a.Hkv;
    kvh = i % a.Hkv;
    rt = g * nb + tb;
  } else {
    kvh = (total - 1 - i) / n_rt;
    rt = (total - 1 - i) % n_rt;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % G::RG;
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t row_base = (int64_t)kvh * rows;
  const uint32_t qsign = a.q_neg ? 0x80008000u : 0u;

  u32x4_t qf[G::NT][G::SD];
  load_q_rows<G>(qf, a.q + (row_base + rt * G::BM) * G::D, min(rows - rt * G::BM, G::BM), rg, lane, qsign);

  // With a history: its normalised output O_h (fp32) and lse_h, i.e. the
  // state m = lse_h (log2 units), l = 1, O = O_h, which the loop continues.
  WaveState<G> ws;
  const bool fresh = a.L_act == 0;
  if (!fresh) {
    // the tile's rows of both buffers as buffer ranges: no branch around the
    // loads, so they do not hold up the first K/V tile loads
    const int nrow = min(rows - rt * G::BM, G::BM);
    const auto ro = make_rsrc(a.ws_o + (row_base + rt * G::BM) * G::D, (uint32_t)nrow * G::D * 4);
    const auto rm = make_rsrc(a.ws_ml + row_base + rt * G::BM, (uint32_t)nrow * 4);
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      const uint32_t lr = (uint32_t)((rg * G::NT + nt) * 32 + l32);
      const bool ok = rt * G::BM + (int)lr < rows;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x4_t x = buf_load16(ro, (lr * G::D + mt * 32 + r4 * 8 + 4 * hh) * 4);
#pragma unroll
          for (int c = 0; c < 4; ++c) ws.o[nt][mt][4 * r4 + c] = __uint_as_float(x[c]);
        }
      const float lse_h = buf_load_f32(rm, lr * 4);
      ws.m[nt] = ok ? lse_h * kLog2e : -INFINITY;
      ws.l[nt] = ok && hh == 0 ? 1.0f : 0.0f;  // the pair sum of the two halves gives l = 1
    }
  }

  CausalMask<G::NT> cm;
  int tmin = 0x3fffffff;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int r = rt * G::BM + (rg * G::NT + nt) * 32 + l32;
    cm.t[nt] = r < rows ? r % a.Lq : 0x3fffffff;  // padding rows: see everything, never written
    tmin = min(tmin, cm.t[nt]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tmin = min(tmin, __shfl_xor(tmin, o, 64));
  cm.t_min = __builtin_amdgcn_readfirstlane(tmin);
  // keys this tile needs: one past its largest token (all of them when its
  // rows span two heads)
  const int first = rt * G::BM, last = min(first + G::BM, rows) - 1;
  const int n_keys = first / a.Lq == last / a.Lq ? last % a.Lq + 1 : a.Lq;
  if constexpr (G::DMA) {  // the current K/V as tile images
    TileImgSrc<G> src;
    src.img = a.img_cur + (int64_t)kvh * a.n_tiles_cur * TileImgSrc<G>::TIMG;
    src.n_tiles = a.n_tiles_cur;
    src.n_keys = n_keys;
    flash_loop_dma<G>(ws, src, qf, smem, a.c_cur, cm, fresh, threadIdx.x);
  } else {
    EncSrc<G, false, false> cs;
    cs.kb = reinterpret_cast<const char *>(a.kcur + (int64_t)kvh * a.Lq * G::D);
    cs.vb = reinterpret_cast<const char *>(a.vcur + (int64_t)kvh * a.Lq * G::D);
    cs.krow = cs.vrow = G::D * 2;
    cs.kstep = cs.vstep = (int64_t)G::NSPLIT * G::BN * G::D * 2;
    cs.n_keys = n_keys;
    cs.mask = nullptr;
    flash_loop<G, false>(ws, cs, qf, smem, a.c_cur, cm, fresh, threadIdx.x);
  }

  prefill_epilogue<G, false>(ws, a, rt, kvh, rg, lane, 1.0f);
}

// ------------------------------------------------------------------ tile images

// Write the bf16 tile images the DMA key loop copies (TileImgSrc): one
// workgroup per (tile, KV head).  Source: the live history of the paged FP8
// cache (e4m3fn -> bf16, exact), or with CUR the current tokens' bf16 K/V
// [Hkv, Lq, D].  Keys past the end are written as zeros.  K reads run along
// each key row (coalesced) and write chunk-major; V is transposed through
// LDS.
template <class G, bool CUR>
__global__ __launch_bounds__(256) void prefill_tile_images_kernel(PrefillLaunch a) {
  constexpr int CH = G::D / 8;                  // 16-byte bf16 chunks per key
  const int t = blockIdx.x, kvh = blockIdx.y;
  const int n_keys = CUR ? a.Lq : a.L_act;
  char *const img = (CUR ? a.img_cur : a.img) + ((int64_t)kvh * (CUR ? a.n_tiles_cur : a.n_tiles) + t) *
                                                    TileImgSrc<G>::TIMG;
  auto src16 = [&](bool is_k, int key, int c) -> u32x4_t {  // 8 bf16 of key `key`, chunk c
    if constexpr (CUR) {
      const __bf16 *p = (is_k ? a.kcur : a.vcur) + ((int64_t)kvh * a.Lq + key) * G::D + c * 8;
      return *reinterpret_cast<const u32x4_t *>(p);
    } else {
      const int32_t phys = a.bt[key / a.bs];
      const uint8_t *p = (is_k ? a.kc : a.vc) + (((int64_t)phys * a.Hkv + kvh) * a.bs + key % a.bs) * G::D + c * 8;
      return PagedSrc<G>::cvt8(*reinterpret_cast<const u32x2_t *>(p));
    }
  };
  for (int i = threadIdx.x; i < G::BN * CH; i += 256) {
    const int k = i / CH, c = i % CH, key = t * G::BN + k;
    const u32x4_t x = key < n_keys ? src16(true, key, c) : u32x4_t{0, 0, 0, 0};
    *reinterpret_cast<u32x4_t *>(img + c * (G::BN * 16) + k * 16) = x;
  }
  // V^T: the tile's rows go through LDS ([key][d] bf16), then thread i
  // writes the image's 16-byte chunk i (consecutive threads, consecutive
  // bytes): k-step i / 2D, d = (i / 2) % D, stored chunk i % 2
  __shared__ u32x4_t vstage[G::BN * CH];
  for (int i = threadIdx.x; i < G::BN * CH; i += 256) {
    const int k = i / CH, c = i % CH, key = t * G::BN + k;
    vstage[i] = key < n_keys ? src16(false, key, c) : u32x4_t{0, 0, 0, 0};
  }
  __syncthreads();
  const uint16_t *vs = reinterpret_cast<const uint16_t *>(vstage);
  for (int i = threadIdx.x; i < G::D * 4; i += 256) {
    const int kk = i / (2 * G::D), d = (i / 2) % G::D, h = (i % 2) ^ G::vt_swz(d);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = vs[G::vt_key(kk, h, 2 * e) * G::D + d] | (uint32_t)vs[G::vt_key(kk, h, 2 * e + 1) * G::D + d] << 16;
    *reinterpret_cast<u32x4_t *>(img + G::KTILE + i * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// ------------------------------------------------------------------ launchers

// BM 128, 8 waves: 4 row groups x 2 key splits, 32-key tiles, 4 waves/SIMD; bf16 K/V copied global -> LDS by
// direct loads (the boundary requires 16-byte aligned bases and strides that are multiples of 8 elements)
using EncGeo = Geo<64, 32, 1, 4, 2, 4, 4, true, 0, false, false, true, true, true>;
// the same with 64-key tiles (half the barriers and per-tile work per key) at the 2-wave register budget and
// 128 KiB of LDS: for grids of at most one workgroup per CU, where neither limit costs occupancy
using EncGeo64 = Geo<64, 64, 1, 4, 2, 4, 2, true, 0, false, false, true, true, true>;
using EncGeoMask = Geo<64, 32, 1, 4, 2, 4, 2, true>;  // masked: register-staged tiles and mask values, 2 waves/SIMD
using EncGeoF32 = Geo<64, 32, 1, 4, 2, 4, 2, true>;   // fp32 inputs: register-staged (converted) tiles
using PrefGeo = Geo<256, 32, 1, 8, 1, 2, 2, false, 3, true>;  // BM 256, 8 waves of 32 rows, 2 waves per SIMD, 3 Q fragments in LDS, PV priority
using PrefImgGeo = Geo<256, 32, 1, 8, 1, 2, 2, false, 0, false, true>;  // the same over bf16 tile images copied by DMA (no staging registers: Q fits in registers; no PV priority)
using PrefCurImgGeo = Geo<256, 32, 1, 8, 1, 2, 2, false, 4, false, true>;  // current tokens over their images: the causal state needs 4 Q fragments in LDS to stay out of scratch

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

// Compute units of the current device (cached per device; 0 if unknown).
static int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// ROPE here rotates the Q rows as they are loaded; K arrives rotated (the
// RoPE pass of rope.hip).
template <int ROPE>
static hipError_t launch_encoder_r(const EncoderLaunch &a, bool f32_in, dim3 grid, hipStream_t stream) {
  if (f32_in)
    return a.mask ? launch_lds<EncGeoF32>(encoder_fwd_kernel<EncGeoF32, true, true, ROPE>, grid, a, stream)
                  : launch_lds<EncGeoF32>(encoder_fwd_kernel<EncGeoF32, true, false, ROPE>, grid, a, stream);
  if (a.mask) return launch_lds<EncGeoMask>(encoder_fwd_kernel<EncGeoMask, false, true, ROPE>, grid, a, stream);
  // 64-key tiles from 1536 keys on (measured at 256 workgroups of 2048 query rows: 1.3% slower at 1024
  // keys, even at 1280, 1-4% faster from 1536 to 4096)
  if ((int)grid.x <= cu_count() && a.Skv >= 1536)
    return launch_lds<EncGeo64>(encoder_fwd_kernel<EncGeo64, false, false, ROPE>, grid, a, stream);
  return launch_lds<EncGeo>(encoder_fwd_kernel<EncGeo, false, false, ROPE>, grid, a, stream);
}

hipError_t launch_encoder(const EncoderLaunch &a, bool f32_in, hipStream_t stream) {
  const int n_qt = (a.Sq + EncGeo::BM - 1) / EncGeo::BM;
  const dim3 grid(n_qt * a.H * a.B);
  static_assert(EncGeo::BM == EncGeoF32::BM && EncGeo::THREADS == EncGeoF32::THREADS, "same launch shape");
  static_assert(EncGeo::BM == EncGeoMask::BM && EncGeo::THREADS == EncGeoMask::THREADS, "same launch shape");
  static_assert(EncGeo::BM == EncGeo64::BM && EncGeo::THREADS == EncGeo64::THREADS, "same launch shape");
  switch (a.rope) {
    case 0: return launch_encoder_r<0>(a, f32_in, grid, stream);
    case 1: return launch_encoder_r<1>(a, f32_in, grid, stream);
    case 2: return launch_encoder_r<2>(a, f32_in, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

int encoder_rows_per_block() { return EncGeo::BM; }

int64_t prefill_tile_image_bytes() { return TileImgSrc<PrefImgGeo>::TIMG; }

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream) {
  const int rows = a.G * a.Lq;
  const int n_rt = (rows + PrefGeo::BM - 1) / PrefGeo::BM;
  static_assert(PrefImgGeo::BM == PrefGeo::BM && PrefImgGeo::BN == PrefGeo::BN, "same tiles");
  const dim3 grid(n_rt * a.Hkv);
  if (a.img && a.L_act > 0) {  // the history through its tile images
    hipLaunchKernelGGL((prefill_tile_images_kernel<PrefImgGeo, false>), dim3(a.n_tiles, a.Hkv), dim3(256), 0, stream,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!a.kcur) return launch_lds<PrefImgGeo>(prefill_paged_kernel<PrefImgGeo, false>, grid, a, stream);
    const hipError_t e2 = launch_lds<PrefImgGeo>(prefill_paged_kernel<PrefImgGeo, true>, grid, a, stream);
    if (e2 != hipSuccess) return e2;
  } else if (!a.kcur) {
    return launch_lds<PrefGeo>(prefill_paged_kernel<PrefGeo, false>, grid, a, stream);
  } else if (a.L_act > 0) {
    const hipError_t e = launch_lds<PrefGeo>(prefill_paged_kernel<PrefGeo, true>, grid, a, stream);
    if (e != hipSuccess) return e;
  }
  if (a.img_cur) {  // the current tokens through their tile images
    static_assert(PrefCurImgGeo::BM == PrefGeo::BM && TileImgSrc<PrefCurImgGeo>::TIMG == TileImgSrc<PrefImgGeo>::TIMG,
                  "same row tiles and tile images");
    hipLaunchKernelGGL((prefill_tile_images_kernel<PrefImgGeo, true>), dim3(a.n_tiles_cur, a.Hkv), dim3(256), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_lds<PrefCurImgGeo>(prefill_current_kernel<PrefCurImgGeo>, grid, a, stream);
  }
  return launch_lds<PrefGeo>(prefill_current_kernel<PrefGeo>, grid, a, stream);
}

int prefill_key_tile() { return PrefGeo::BN; }
int prefill_rows_per_block() { return PrefGeo::BM; }

}  // namespace mi355
