// GQA single-token decode, head_dim 256 or 512, split-K ("flash-decode") +
// combine, over the whole cache or over a per-sequence key range.
//
// head_dim>128 (256/512) GQA Flash-Decode NKI Kernel for AWS Trainium,
// "Input contract" fixes the operands (q [B,Hq,1,D], k/v [B,Hkv,S_ctx,D],
// additive 0/-inf mask [B,1,1,S_ctx], softmax_scale, num_kv_groups); its
// "Perf caveat" and "Future performance follow-on" note that one program
// re-streaming the whole cache is bandwidth-starved and that the KV stream
// should be sharded over many programs, and that sliding-window layers need
// only the most recent window of keys.  Here every (batch, KV head, chunk of
// 64 keys) is its own workgroup (the highest chunks dispatched first), the
// G query heads of a KV head share the one pass over its K/V, and a second
// kernel merges the chunk partials.  With
// a key range the grid spans only the chunks the widest range can touch,
// counted from each sequence's own first key (a windowed gather: keys before
// the window are never fetched and get no workgroup).  The introduction of
// the same page names the two head sizes: 256 on sliding-window layers, 512
// on global ones.
//
// Split kernel, per workgroup (4 waves of kDecNG groups of 16 keys; with more
// than one group the loads of group g+1 are in flight while group g is
// computed, and an online softmax runs across the groups):
//   QK^T : v_mfma_f32_16x16x32_bf16 with the 16 keys on M and the G query
//          heads on N (padded to 16), K streamed straight from HBM into the
//          A operand (64 contiguous bytes per key per load);
//   mask : additive, in log2 units; keys it removes are never fetched (their
//          buffer offsets fall out of range), a wave with no live key skips
//          the loads;
//   softmax: in the MFMA's score layout, one head per 16-lane column (four
//          exp2 per lane; the group's max and sum over the head's four
//          lanes), P to LDS;
//   PV   : on the VALU, each lane owning D/64 of the D output columns, V read
//          with 2D contiguous bytes per key per wave;
//   merge: the 4 wave partials combine through LDS; the chunk partial
//          (m, l in log2 units, unnormalised o) goes to the workspace.
// Combine kernel, per (b, query head): M = max m_c, L = sum 2^(m_c-M) l_c,
//   o = sum 2^(m_c-M) o_c / L over the chunks in index order (deterministic).
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace mi355 {

constexpr int kDecKW = 16;                      // keys per group (one 16-key MFMA block)
constexpr int kDecNG = 1;                       // groups per wave
constexpr int kDecWaves = 4;                    // waves per workgroup
constexpr int kDecChunk = kDecWaves * kDecNG * kDecKW;  // keys per workgroup
constexpr int kDecGmax = 8;                     // query heads per KV head supported
constexpr uint32_t kOOB = 0x80000000u;          // buffer offset past any range: the load returns zeros
// K and V are read exactly once: non-temporal loads (cache policy "nt").  On
// this part they stream at about twice the rate of default-policy loads.
constexpr int kNT = 2;

// Raw buffer resource over [base, base + bytes) (uniform arguments; see the
// flash kernels for why readfirstlane).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Max and sum over the four lanes l % 16 + 16 q of a 16-lane column (lane ^ 16,
// then lane ^ 32); all four receive the same bits.
__device__ __forceinline__ float dec_quad_max(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float dec_quad_sum(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Per-lane V slice: D/64 bf16 columns of one key (4 -> 8 bytes, 8 -> 16).
template <int D> struct DecV;
template <> struct DecV<256> {
  typedef u32x2_t type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
  }
};
template <> struct DecV<512> {
  typedef u32x4_t type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
  }
};

// One group of 16 keys in registers: K as the A operand of the QK MFMA
// (lane l: key l%16, d = 32s + 8(l/16) .. +7) and V as 16 rows of the lane's
// D/64 output columns.
template <int D>
struct DecStage {
  u32x4_t k[D / 32];
  typename DecV<D>::type v[kDecKW];
};

// Issue the loads of group g (keys g*16 .. g*16+15 of the wave); keys that
// are not live get an out-of-range offset and are never fetched.
template <int D>
__device__ __forceinline__ void dec_load(DecStage<D> &st, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         uint64_t live, int g, int lane) {
  const int gq = lane & 15, quad = lane >> 4;
  const int kk = g * kDecKW + gq;
  const uint32_t koff = ((live >> kk) & 1) ? kk * (D * 2) + 16 * quad : kOOB;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    st.k[s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * s, 0, kNT));
#pragma unroll
  for (int j = 0; j < kDecKW; ++j) {
    const int kj = g * kDecKW + j;
    const uint32_t voff = ((live >> kj) & 1) ? kj * (D * 2) + (D / 32) * lane : kOOB;
    st.v[j] = DecV<D>::load(rv, voff);
  }
}

// Key range of sequence b: [beg, end) clamped to [0, S_ctx], then cut to its
// last max_keys keys; chunk 0 of the sequence starts at beg rounded down to
// a chunk boundary.
struct DecRange {
  int beg, end, base;
};
__device__ __forceinline__ DecRange dec_range(const DecodeLaunch &a, int b) {
  int end = a.S_ctx, beg = 0;
  if (a.key_end) end = min(max(a.key_end[b], 0), a.S_ctx);
  if (a.key_begin) beg = min(max(a.key_begin[b], 0), end);
  beg = max(beg, end - a.max_keys);
  return DecRange{beg, end, beg - beg % kDecChunk};
}

// The accumulator of one query head: the lane's D/64 output columns.
template <int D> struct DecAcc { float x[D / 64]; };

// Register budget (waves per SIMD): at head_dim 256, 5 waves fit up to four
// query heads per KV head (at most 96 VGPRs, no scratch); eight take the
// 4-wave budget.
template <int D, int G> constexpr int dec_waves_per_eu() { return D == 256 ? (G >= 8 ? 4 : 5) : 2; }

template <int D, int G>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<D, G>())))
void decode_split_kernel(DecodeLaunch a) {
  constexpr int KW = kDecKW, NW = kDecWaves, NG = kDecNG, WK = NG * KW;  // WK: keys per wave
  constexpr int CPL = D / 64;                                             // output columns per lane
  static_assert(WK <= 64, "one liveness bit per lane");
  // LDS: each wave's copy of the G query rows and its tile of P (used in
  // the key loop), then the wave partials of the merge.  When the three
  // together would cap occupancy the merge buffer reuses the first two,
  // behind one more barrier.
  constexpr int QS_B = NW * G * D * 2, PL_B = NW * G * KW * 4, RO_B = NW * G * D * 4;
  constexpr bool ALIAS = QS_B + PL_B + RO_B > 48 * 1024;
  constexpr int SMEM_B = ALIAS ? (QS_B + PL_B > RO_B ? QS_B + PL_B : RO_B) : QS_B + PL_B + RO_B;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_B];
  __shared__ float red_ml[NW][G][2];
  auto qs = reinterpret_cast<__bf16(*)[G][D]>(smem);
  auto pl = reinterpret_cast<float(*)[G][KW]>(smem + QS_B);
  auto red_o = reinterpret_cast<float(*)[G][D]>(smem + (ALIAS ? 0 : QS_B + PL_B));

  // One-dimensional grid, chunk-major with the last chunks first: the chunks
  // that most sequences leave empty (the highest) are dispatched first and
  // exit early, and the final workgroups are the all-live first chunks of
  // every (batch, KV head), which finish together.  A timeline of the
  // workgroups showed the (batch-major) order ending in a long tail of the
  // last batch's chunks.  At head_dim 512 (3 waves per SIMD, so fewer
  // workgroups resident, each with twice the bytes) the chunk order
  // alternates between the highest and the lowest remaining chunk instead,
  // so the K/V stream starts with the first workgroups (measured faster
  // there, slower at 256).
  const int np = a.Hkv * a.B, lin = blockIdx.x, j = lin / np;
  const int chunk = (D == 512 && (j & 1)) ? j / 2 : a.n_chunks - 1 - (D == 512 ? j / 2 : j);
  const int kvh = (lin % np) % a.Hkv, b = (lin % np) / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const DecRange R = dec_range(a, b);
  const float *mrow = a.mask ? a.mask + (int64_t)b * a.S_ctx : nullptr;
  const int64_t part0 = ((int64_t)b * a.Hq + (int64_t)kvh * G) * a.n_chunks + chunk;  // head g adds g*n_chunks
  const int ckey0 = R.base + chunk * kDecChunk;  // first key of the chunk
  const int key0 = ckey0 + wave * WK;

  // Every wave reads the mask of the whole chunk (lane l: key l of the chunk,
  // log2 units, -inf where removed or outside the range) and votes: a chunk
  // with no live key writes its empty statistics and exits without touching
  // K/V or the LDS (every wave takes the same branch, no barrier needed).
  // Keys outside the range never read the mask.
  static_assert(kDecChunk <= 64, "one chunk key per lane");
  float mk_lane = -INFINITY;
  if (lane < kDecChunk) {
    const int key = ckey0 + lane;
    const float mv = (key >= R.beg && key < R.end) ? (mrow ? mrow[key] : 0.0f) : -INFINITY;
    mk_lane = mv == -INFINITY ? -INFINITY : mv * kLog2e;
  }
  const uint64_t live_chunk = __ballot(mk_lane != -INFINITY);
  if (live_chunk == 0) {
    if (tid < G) {
      const int64_t part = part0 + (int64_t)tid * a.n_chunks;
      a.ws_ml[part * 2 + 0] = -INFINITY;
      a.ws_ml[part * 2 + 1] = 0.0f;
    }
    return;
  }
  const uint64_t live = (live_chunk >> (wave * WK)) & ((WK == 64) ? ~0ull : ((1ull << WK) - 1));

  const int gq = lane & 15, quad = lane >> 4;
  // Softmax state of the lane's head (lane % 16, in the score layout of the
  // QK MFMA; the same in all four lanes of a head) and the G heads' partial
  // outputs over the lane's columns.
  float m_l = -INFINITY, l_l = 0.0f;
  DecAcc<D> o[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[g].x[c] = 0.0f;

  if (live != 0) {
    const int64_t row0 = ((int64_t)b * a.Hkv + kvh) * a.S_ctx + key0;
    const uint32_t span = (uint32_t)max(min(WK, R.end - key0), 0) * (D * 2);
    const auto rk = dec_rsrc(a.k + row0 * D, span), rv = dec_rsrc(a.v + row0 * D, span);
    // The G query rows (G * 2D bytes) go into this wave's LDS slice: the
    // q^T B-operand fragments are read from there right before their MFMAs,
    // which keeps them out of the registers.  q's loads are issued first and
    // written to LDS after the first group's K/V loads are issued, so the
    // K/V stream does not wait for q's round trip.
    constexpr int QL = (G * D * 2 + 1023) / 1024;  // 16-byte q loads per lane
    const auto rq = dec_rsrc(a.q + ((int64_t)b * a.Hq + (int64_t)kvh * G) * D, G * D * 2);
    u32x4_t qv[QL];
#pragma unroll
    for (int i = 0; i < QL; ++i)  // offsets past the G rows read zeros and are not written
      qv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (lane + 64 * i) * 16, 0, 0));
    DecStage<D> st[NG < 2 ? 1 : 2];
    dec_load<D>(st[0], rk, rv, live, 0, lane);
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const uint32_t off = (lane + 64 * i) * 16;
      if (off < G * D * 2) *reinterpret_cast<u32x4_t *>(reinterpret_cast<char *>(&qs[wave][0][0]) + off) = qv[i];
    }

#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      if (grp + 1 < NG) {
        // issue group grp+1 now, not earlier: the pinned copy of the liveness
        // mask keeps the compiler from hoisting every group's loads to the top
        uint64_t live_n = live;
        asm volatile("" : "+s"(live_n));
        dec_load<D>(st[(grp + 1) & 1], rk, rv, live_n, grp + 1, lane);
      }
      const DecStage<D> &cs = st[NG < 2 ? 0 : grp & 1];
      // q^T fragment: lane l holds q[g = l%16][32s + 8(l/16) .. +7], zero for g >= G
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's copy of q is in LDS
      __builtin_amdgcn_wave_barrier();
      const char *qrow = reinterpret_cast<const char *>(&qs[wave][gq < G ? gq : 0][0]) + 16 * quad;
      f32x4_t s4 = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const u32x4_t qv = *reinterpret_cast<const u32x4_t *>(qrow + 64 * s);
        s4 = mfma16(as_bf16x8(cs.k[s]), as_bf16x8(gq < G ? qv : u32x4_t{0, 0, 0, 0}), s4);
      }
      // lane l holds S^T[key = 4*(l/16) + i][head g = l%16]: scale and mask,
      // then the online softmax of head l%16 in this layout (four exp2 per
      // lane; the group max and sum run over the head's four lanes), and P
      // to LDS for the PV
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mv = __shfl(mk_lane, wave * WK + grp * KW + 4 * quad + i);
        s4[i] = mv == -INFINITY ? -INFINITY : __builtin_fmaf(s4[i], a.c, mv);
      }
      const float mg = dec_quad_max(fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3])));
      const float m_new = fmaxf(m_l, mg);
      const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_l - m_new);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;  // a head with no live key yet: p = 0
      m_l = m_new;
      f32x4_t p4;
#pragma unroll
      for (int i = 0; i < 4; ++i) p4[i] = fast_exp2(s4[i] - m_use);
      l_l = l_l * alpha + dec_quad_sum((p4[0] + p4[1]) + (p4[2] + p4[3]));
      if (gq < G) *reinterpret_cast<f32x4_t *>(&pl[wave][gq][4 * quad]) = p4;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      // PV on the VALU for each head, after its rescale (alpha of head g from lane g)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), g));
        DecAcc<D> acc;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc.x[c] = o[g].x[c] * ag;
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const float pj = pl[wave][g][j];
#pragma unroll
          for (int w = 0; w < CPL / 2; ++w) {
            acc.x[2 * w] += pj * bf16_lo(cs.v[j][w]);
            acc.x[2 * w + 1] += pj * bf16_hi(cs.v[j][w]);
          }
        }
        o[g] = acc;
      }
      __builtin_amdgcn_wave_barrier();  // pl is rewritten by the next group
    }
  }

  float m[G], l[G];  // per head, from the head's lane
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_l), g));
    l[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_l), g));
  }

  // Merge the wave partials (fixed order) and write the chunk partial.
  if (ALIAS) __syncthreads();  // every wave is done with its q copy and P tile
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int c = 0; c < CPL; c += 4)
      *reinterpret_cast<f32x4_t *>(&red_o[wave][g][CPL * lane + c]) =
          f32x4_t{o[g].x[c], o[g].x[c + 1], o[g].x[c + 2], o[g].x[c + 3]};
    if (lane == 0) {
      red_ml[wave][g][0] = m[g];
      red_ml[wave][g][1] = l[g];
    }
  }
  __syncthreads();
  // thread t handles (head, column) pairs t, t + 256, ... of the G x D partial
  static_assert((G * D) % (64 * NW) == 0, "whole rounds of the merge");
#pragma unroll
  for (int i0 = 0; i0 < G * D; i0 += 64 * NW) {
    const int g = (i0 + tid) / D, col = (i0 + tid) % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_ml[w][g][0]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = fast_exp2(red_ml[w][g][0] - Mu);
      L += red_ml[w][g][1] * sw;
      acc += red_o[w][g][col] * sw;
    }
    const int64_t part = part0 + (int64_t)g * a.n_chunks;
    if (M != -INFINITY) a.ws_o[part * D + col] = acc;
    if (col == 0) {
      a.ws_ml[part * 2 + 0] = M;
      a.ws_ml[part * 2 + 1] = L;
    }
  }
}

// Combine: one 64-thread workgroup per (batch, query head, 64-column slice),
// 64 chunks per round.  Lane c reads chunk c's statistics; the max and the
// weighted sum of l are wave reductions; every lane issues its column's loads
// for all 64 chunks at once and weights them with the chunk weight broadcast
// from lane c.  Dead chunks (m_c = -inf, partial never written) get an
// out-of-range offset, so their partials are never fetched; they and chunks
// whose weight underflows are selected away, not branched around.  The chunk
// order is fixed, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeLaunch a) {
  const int slice = blockIdx.x, hq = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int64_t p0 = ((int64_t)b * a.Hq + hq) * a.n_chunks;
  const int d = slice * 64 + lane;
  const auto ro = dec_rsrc(a.ws_o + p0 * D, (uint32_t)a.n_chunks * D * 4);  // this head's chunk partials
  float M = -INFINITY, L = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 64) {
    const int nc = min(64, a.n_chunks - c0);
    const int64_t pc = p0 + c0 + (lane < nc ? lane : 0);
    const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(a.ws_ml + pc * 2);
    const float mc = lane < nc ? ml[0] : -INFINITY;
    const uint64_t alive = __ballot(mc != -INFINITY);  // bit i: chunk c0 + i has a partial
    float oc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
      oc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             ro, ((alive >> i) & 1) ? (uint32_t)((c0 + i) * D + d) * 4 : kOOB, 0, 0));
    float mcp = mc;
    asm volatile("" : "+v"(mcp));  // the reductions below run while the loads are in flight
    const float Mb = fmaxf(M, wave_max(mcp));
    const float Mu = Mb == -INFINITY ? 0.0f : Mb;
    const float w = mc == -INFINITY ? 0.0f : fast_exp2(mc - Mu);
    const float rs = M == -INFINITY ? 0.0f : fast_exp2(M - Mu);  // rescale of the running sums
    L = L * rs + wave_sum(w > 0.0f ? ml[1] * w : 0.0f);
    acc *= rs;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i));
      acc += wi > 0.0f ? oc[i] * wi : 0.0f;
    }
    M = Mb;
  }
  const float r = L > 0.0f ? acc / L : 0.0f;
  a.out[((int64_t)b * a.Hq + hq) * D + d] = (__bf16)r;
}

template <int D>
static hipError_t launch_decode_d(const DecodeLaunch &a, hipStream_t stream) {
  const dim3 grid(a.n_chunks * a.Hkv * a.B), block(64 * kDecWaves);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(D / 64, a.Hq, a.B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
  switch (a.D) {
    case 256: return launch_decode_d<256>(a, stream);
    case 512: return launch_decode_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Scratch of the allocation-free decode entry point: the chunk partials live
// in this file-scope device array instead of a caller workspace.  Each GPU
// holds its own copy at its own address (found once per device with
// hipGetSymbolAddress; in host code the array's name is only a stand-in and
// is never passed to a kernel).  Every call on one GPU shares it.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(hipStream_t stream, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *per_device[kMaxDevices];
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

int decode_chunk_keys() { return kDecChunk; }
int decode_max_groups() { return kDecGmax; }

}  // namespace mi355
