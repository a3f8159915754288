// a4 - gather attention over the position buffer.
//
// The arex-research.com article (section on the four optimisations, item 3)
// describes a sparse attention kernel for normal decode and MTP verify with
// BF16 queries and BF16 or FP8 E4M3 KV.  This is a gfx950 design for the same
// contract.
//
// Work unit: (query, KV head, split of the position buffer), the position in
// a 3-D grid dispatched query fastest and split slowest - or, for a batch of
// several requests with fewer than 512 units, item w of a longest-first work
// list (AttnPlan) in a 1-D grid, the splits sized from the batch's total
// positions so that long units get more workgroups than short ones.  A wave
// takes 32 gathered positions per step and serves the whole GQA group of that KV head
// (up to 16 query heads) at once on bf16 MFMA 16x16x32:
//   S^T[pos][head] = K[pos][:] . Q[head][:]      (2 tiles x 4 MFMAs)
//   O^T[dim][head] += V^T[dim][pos] P^T[pos][head]  (8 MFMAs each for the BF16
//                                                    high and low parts of P)
// The GQA group is the 16-column side of the tile; the gathered positions
// are the dense side.  The position order inside the k dimension of the PV
// product is chosen so that each lane's P values come straight out of the
// S^T accumulator registers, and each lane gathers exactly the V rows its own
// P values need (16 contiguous bytes per row), repacked with byte permutes -
// no LDS round trip.  FP8 E4M3FN rows are widened exactly to BF16 with the
// hardware converter; the per-head K scale folds into the softmax scale and
// the V scale into the final normalisation.
//
// Softmax is online per wave (running reference max, moved lazily, and sum in
// the log2 domain), the 4 waves of a workgroup merge in LDS, and when a unit
// is split over several workgroups the last one to finish merges the
// partials (an arrival counter in the workspace, one 128-byte line per unit,
// reset to zero by that last workgroup).  Partials travel through
// device-scope buffer stores and loads that bypass the per-XCD caches, so the
// hand-off needs no cache flush or invalidation.  In the large-batch
// (non-temporal) kernels the K rows of a step go through LDS by
// direct-to-LDS loads of whole lines; V always goes to registers.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kOStride = QSA_HEAD_DIM + 4;   // padded LDS row of one head's output
// Device-scope 16-byte loads and stores through a raw buffer descriptor of a
// split-partial region.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f32x4 load_coherent(__amdgpu_buffer_rsrc_t r, int float_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, float_off * 4, 0, kCpolDevice);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int float_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, float_off * 4, 0, kCpolDevice);
}
__device__ __forceinline__ float load_coherent_f32(__amdgpu_buffer_rsrc_t r, int float_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, float_off * 4, 0, kCpolDevice));
}
__device__ __forceinline__ void store_coherent_f32(__amdgpu_buffer_rsrc_t r, int float_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, float_off * 4, 0, kCpolDevice);
}
constexpr int kMaxHeads = 8 * kMaxSplitChunks;   // block heads of one split (8 per chunk)
constexpr float kRescaleSlack = 8.f;     // log2 headroom of the softmax reference maximum
constexpr int kNtMinUnits = 256;         // (query, KV head) units from which K/V loads are non-temporal

struct AttnParams {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const int32_t* pos;
  const int32_t* n_pos;
  void* out;
  float* part;
  uint32_t* counters;
  uint32_t* err;            // error word (QSA_ERROR_* bits), or nullptr
  int num_q, width, num_q_heads, num_kv_heads, group;
  int run_heads;            // pos holds one slot per 4-slot run (rows of width entries)
  float sm_scale_log2;
  int splits, cps;
  const int32_t* plan;      // the ragged batch's work list (AttnPlan), or nullptr: the grid is (q, KV head, split)
};

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4 FP8 E4M3FN bytes -> 4 BF16 (exact), as 2 packed dwords (low bytes first).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool kFp8> struct VRaw { typedef u32x4 type; };   // 8 BF16 of one V row
template <> struct VRaw<true> { typedef u32x2 type; };      // 8 FP8 of one V row

// First of the 8 dimensions that step kk of the S = K Q^T chain contracts in
// lane group kg.  A K load instruction w reads bytes 64w + 16kg .. 64w + 16kg
// + 15 of each of its 16 rows, so the four lane groups read 64 contiguous
// bytes of a row together.  BF16: load w holds dimensions 32w + 8kg .. + 7,
// step kk = w.  FP8: load w holds dimensions 64w + 16kg .. + 15, the first
// half for step 2w, the second for step 2w + 1.  The query uses the same map.
template <bool kFp8>
__device__ __forceinline__ int kdim(int kk, int kg) {
  return kFp8 ? 64 * (kk >> 1) + 16 * kg + 8 * (kk & 1) : 32 * kk + 8 * kg;
}

// K/V bytes of one 32-position chunk as one lane holds them.  With kKL the
// chunk's K rows go to LDS instead (see KLds) and k is unused.
template <bool kFp8, bool kKL>
struct ChunkRaw {
  u32x4 k[kKL ? 1 : 2][kFp8 ? 2 : 4];   // K rows 16t + j: 16 bytes at 64w + 16kg (see kdim)
  typename VRaw<kFp8>::type v[8];       // V rows 16t + 4kg + rr (e = 4t + rr): dims 8j .. 8j+7
  uint32_t vmask;                       // bit e: V / score position e holds a valid slot
};

// K rows of a chunk in LDS: 32 rows of 128 (FP8) or 256 (BF16) bytes, row
// r's 16-byte piece p stored at slot p XOR kswz(r).  Direct-to-LDS loads
// put lane l's 16 bytes at byte 16l of the instruction's 1 KiB, so an
// instruction moves 8 (FP8) or 4 (BF16) whole rows and each aligned group of
// 8 lanes fetches one whole 128-byte line; the swizzle then makes the MFMA
// operand reads (16 rows, one piece each) hit 16 different bank groups.
// LDS reads issued as inline assembly that waits for its own results.  The
// compiler treats any LDS read that follows a direct-to-LDS load as possibly
// reading that load's data and waits for every vector-memory operation in
// flight, which would drain the next chunk's prefetch; the reads here touch
// only LDS the loads in flight do not write (block heads, or a K buffer whose
// loads were waited for explicitly).
__device__ __forceinline__ void lds_read_2x_b128(u32x4& a, u32x4& b, const uint8_t* pa, const uint8_t* pb) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"((__attribute__((address_space(3))) const uint8_t*)pa),
                 "v"((__attribute__((address_space(3))) const uint8_t*)pb));
}

template <bool kFp8> struct KLds {
  static constexpr int kRowBytes = kFp8 ? 128 : 256;
  static constexpr int kBytes = 32 * kRowBytes;              // one chunk
  static constexpr int kLoads = kBytes / 1024;               // load instructions per chunk
  __device__ static constexpr int swz(int r) { return kFp8 ? (r >> 1) & 7 : r & 15; }
};

// Block heads of one chunk: the position buffer is made of runs of 4
// consecutive slots (one 4-token block each), so entry i is head(i & ~3) + (i & 3).
struct ChunkHeads {
  int k[8];   // heads of the blocks holding K rows 16t + j (registers), or the K rows this lane moves to LDS (load i)
  int v[2];   // heads of the blocks holding V rows 16t + 4kg + rr
};

// Block heads of chunk c from the workgroup's LDS copy (heads_s[8 * (c - c0) + b]
// is the slot of position 32c + 4b).  LDS reads do not join the in-order
// vector-memory counter, so they never force a wait on K/V loads in flight.
template <bool kFp8, bool kKL>
__device__ __forceinline__ ChunkHeads lds_heads(const int* heads_s, int c_rel, int cps, int lane, int j, int kg) {
  constexpr int kRowsPerLoad = 1024 / KLds<kFp8>::kRowBytes;
  constexpr int kLanesPerRow = KLds<kFp8>::kRowBytes / 16;
  c_rel = min(c_rel, cps - 1);          // chunks past the split only issue masked loads
  if (!kKL) {
    ChunkHeads h;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      h.k[t] = heads_s[8 * c_rel + 4 * t + (j >> 2)];
      h.v[t] = heads_s[8 * c_rel + 4 * t + kg];
    }
    return h;
  }
  u32x4 a, b;                           // the chunk's 8 block heads
  lds_read_2x_b128(a, b, reinterpret_cast<const uint8_t*>(heads_s + 8 * c_rel),
                   reinterpret_cast<const uint8_t*>(heads_s + 8 * c_rel + 4));
  ChunkHeads h;
  const bool odd = lane >> 5;
  // block of K row kRowsPerLoad * i + lane / kLanesPerRow: FP8 loads cover
  // blocks 2i, 2i+1 (lane halves), BF16 loads one block each
  if (kRowsPerLoad == 8) {
    h.k[0] = (int)(odd ? a.y : a.x);
    h.k[1] = (int)(odd ? a.w : a.z);
    h.k[2] = (int)(odd ? b.y : b.x);
    h.k[3] = (int)(odd ? b.w : b.z);
  } else {
    h.k[0] = (int)a.x; h.k[1] = (int)a.y; h.k[2] = (int)a.z; h.k[3] = (int)a.w;
    h.k[4] = (int)b.x; h.k[5] = (int)b.y; h.k[6] = (int)b.z; h.k[7] = (int)b.w;
  }
  // V rows 16t + 4kg + rr sit in block 4t + kg
  h.v[0] = (int)((kg & 2) ? ((kg & 1) ? a.w : a.z) : ((kg & 1) ? a.y : a.x));
  h.v[1] = (int)((kg & 2) ? ((kg & 1) ? b.w : b.z) : ((kg & 1) ? b.y : b.x));
  (void)kLanesPerRow;
  return h;
}

// Load of one K/V piece; kNt marks it non-temporal (streamed past the caches).
template <bool kNt, class T>
__device__ __forceinline__ T kv_load(const uint8_t* p) {
  if constexpr (kNt) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

// Issue the K/V loads of the chunk starting at position `base`.  Positions at
// or past `npos` (all of them when the chunk is past the end) read the first
// slot instead and are masked out, so the issue never needs a branch.
template <bool kFp8, bool kNt, bool kKL>
__device__ __forceinline__ void issue_chunk(ChunkRaw<kFp8, kKL>& ch, uint8_t* klds, const ChunkHeads& h, int base,
                                            int npos, int slot0, const uint8_t* kbase, const uint8_t* vbase,
                                            uint32_t row_stride, int lane, int j, int kg) {
  constexpr int EB = kFp8 ? 1 : 2;
  constexpr int kRowsPerLoad = 1024 / KLds<kFp8>::kRowBytes;
  constexpr int kLanesPerRow = KLds<kFp8>::kRowBytes / 16;
  if (kKL) {
#pragma unroll
    for (int i = 0; i < KLds<kFp8>::kLoads; ++i) {
      const int row = kRowsPerLoad * i + lane / kLanesPerRow;
      const int piece = (lane % kLanesPerRow) ^ KLds<kFp8>::swz(row);
      const uint32_t slot = (uint32_t)(base + row < npos ? h.k[i] + (row & 3) : slot0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kbase + (uint64_t)slot * row_stride + 16 * piece),
          (__attribute__((address_space(3))) void*)(klds + 1024 * i), 16, 0, kNt ? 2 : 0);
    }
  } else {
    const uint8_t* kl = kbase + 16 * kg;      // this lane's bytes inside a K row: 64w + 16kg
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = base + 16 * t + j;
      const uint32_t slot = (uint32_t)(i < npos ? h.k[t] + (j & 3) : slot0);
      const uint8_t* kr = kl + (uint64_t)slot * row_stride;
#pragma unroll
      for (int w = 0; w < (kFp8 ? 2 : 4); ++w) ch.k[t][w] = kv_load<kNt, u32x4>(kr + 64 * w);
    }
  }
  const uint8_t* vl = vbase + j * 8 * EB;     // this lane's bytes inside a V row
  uint32_t vm = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = e >> 2, rr = e & 3;
    const int i = base + 16 * t + 4 * kg + rr;
    const bool valid = i < npos;
    vm |= (uint32_t)valid << e;
    const uint32_t slot = (uint32_t)(valid ? h.v[t] + rr : slot0);
    ch.v[e] = kv_load<kNt, typename VRaw<kFp8>::type>(vl + (uint64_t)slot * row_stride);
  }
  ch.vmask = vm;
}

template <bool kFp8, bool kKL>
__device__ __forceinline__ void compute_chunk(const ChunkRaw<kFp8, kKL>& ch, const uint8_t* klds,
                                              const bf16x8 (&qb)[4], float sl2, float& m_run, float& l_run,
                                              f32x4 (&o)[8], int j, int kg) {
  // K operand (A): step kk takes the 8 dimensions kdim(kk, kg) of row 16t + j,
  // the 16-byte piece 64w + 16kg of the row (w = kk for BF16, kk / 2 for FP8).
  u32x4 kraw[2][kFp8 ? 2 : 4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (kKL) {
      const int row = 16 * t + j;
      const uint8_t* kr = klds + KLds<kFp8>::kRowBytes * row;
#pragma unroll
      for (int w = 0; w < (kFp8 ? 2 : 4); w += 2)
        lds_read_2x_b128(kraw[t][w], kraw[t][w + 1], kr + 16 * ((4 * w + kg) ^ KLds<kFp8>::swz(row)),
                         kr + 16 * ((4 * w + 4 + kg) ^ KLds<kFp8>::swz(row)));
    } else {
#pragma unroll
      for (int w = 0; w < (kFp8 ? 2 : 4); ++w) kraw[t][w] = ch.k[kKL ? 0 : t][w];
    }
  }
  bf16x8 ka[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (kFp8) {
      const uint32_t ws[8] = {kraw[t][0].x, kraw[t][0].y, kraw[t][0].z, kraw[t][0].w,
                              kraw[t][kFp8 ? 1 : 0].x, kraw[t][kFp8 ? 1 : 0].y, kraw[t][kFp8 ? 1 : 0].z,
                              kraw[t][kFp8 ? 1 : 0].w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x2 lo = fp8x4_to_bf16x4(ws[2 * kk]), hi = fp8x4_to_bf16x4(ws[2 * kk + 1]);
        ka[t][kk] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka[t][kk] = __builtin_bit_cast(bf16x8, kraw[t][kk & (kFp8 ? 1 : 3)]);
    }
  }
  // V rows as 8 bf16 each.
  u32x4 vr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (kFp8) {
      const u32x2 lo = fp8x4_to_bf16x4(ch.v[e].x), hi = fp8x4_to_bf16x4(ch.v[e].y);
      vr[e] = u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      vr[e] = ch.v[e];
    }
  }

  // S^T = K Q^T: accumulator row kg*4 + rr = position 16t + 4kg + rr, column j = head.
  f32x4 sacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][kk], qb[kk], sacc[t], 0, 0, 0);
  }
  float sv[8];
  float mloc = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sv[e] = ((ch.vmask >> e) & 1u) ? sacc[e >> 2][e & 3] * sl2 : -INFINITY;
    mloc = fmaxf(mloc, sv[e]);
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
  // Lazy rescaling: the reference maximum only moves when a score exceeds it by
  // more than 2^kRescaleSlack, so weights stay <= 2^kRescaleSlack and the O
  // accumulators are rescaled a handful of times per wave, not every chunk.
  if (__ballot(mloc > m_run + kRescaleSlack)) {
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = o[u] * alpha;
    m_run = m_new;
  }
  // P = P_hi + P_lo, both BF16: the PV product then carries ~16 bits of P.
  uint32_t ph[4], plo[4];
  float psum = 0.f;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const float p0 = __builtin_amdgcn_exp2f(sv[2 * e2] - m_run), p1 = __builtin_amdgcn_exp2f(sv[2 * e2 + 1] - m_run);
    ph[e2] = pack_bf16x2(p0, p1);
    plo[e2] = pack_bf16x2(p0 - bf16lo_to_f32(ph[e2]), p1 - bf16hi_to_f32(ph[e2]));
    psum += p0 + p1;
  }
  l_run += psum;
  const bf16x8 pb_hi = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
  const bf16x8 pb_lo = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});

  // O^T += V^T P^T; tile u covers dims 8i + u for accumulator row i.
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t selb = (u & 1) ? 0x07060302u : 0x05040100u;
    u32x4 a;
    a.x = perm_b32(vr[1][u >> 1], vr[0][u >> 1], selb);
    a.y = perm_b32(vr[3][u >> 1], vr[2][u >> 1], selb);
    a.z = perm_b32(vr[5][u >> 1], vr[4][u >> 1], selb);
    a.w = perm_b32(vr[7][u >> 1], vr[6][u >> 1], selb);
    const bf16x8 va = __builtin_bit_cast(bf16x8, a);
    o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_hi, o[u], 0, 0, 0);
    o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_lo, o[u], 0, 0, 0);
  }
}

// Maximum / sum over the 32 lanes of the wave half this lane is in (every
// lane of the half gets it).
__device__ __forceinline__ float half32_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  const float lo = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)));
  const float hi = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
  return lane_id() >= 32 ? hi : lo;
}
__device__ __forceinline__ float half32_sum(float v) {
  v = row16_sum(v);
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return lane_id() >= 32 ? hi : lo;
}

// Four consecutive outputs (element oi onwards, oi a multiple of 4) as FP32
// or BF16 (nearest-even conversion).
template <bool kOutBf16>
__device__ __forceinline__ void store_out(void* out, int64_t oi, f32x4 v) {
  if (kOutBf16) {
    const bf16x2 a = bf16x2{(__bf16)v.x, (__bf16)v.y}, b = bf16x2{(__bf16)v.z, (__bf16)v.w};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(out) + oi) =
        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oi) = v;
  }
}

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations are outstanding / until all LDS operations are done.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLds = 0xC07F;

constexpr int kAttnThreads = 64 * kAttnWaves;


template <bool kFp8, bool kOutBf16, bool kNt, bool kPlan = false>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  constexpr int D = QSA_HEAD_DIM;
  constexpr int EB = kFp8 ? 1 : 2;            // bytes per KV element
  using KL = KLds<kFp8>;
  // The waves' K chunk buffers (two separate arrays, so that the compiler can
  // tell the direct-to-LDS loads into one from the reads of the other).
  __shared__ __attribute__((aligned(16))) uint8_t kbuf_a[kAttnWaves][KL::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kbuf_b[kAttnWaves][kFp8 ? KL::kBytes : 16];
  __shared__ float o_s[kAttnWaves][16][kOStride];
  __shared__ float m_s[kAttnWaves][16], l_s[kAttnWaves][16];
  __shared__ __attribute__((aligned(16))) int heads_s[kMaxHeads];
  __shared__ int s_last;

  // Grid (query, KV head, split), dispatched query fastest and split
  // slowest: the last split of every unit, which holds only the few
  // positions past the last full 4-chunk group, is dispatched last, so when
  // the grid has more workgroups than the chip has CUs it is those nearly
  // empty workgroups that share a CU with another.
  const int Hkv = p.num_kv_heads;
  int q = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int j = lane & 15, kg = lane >> 4;
  const int G = p.group;
  const bool hvalid = j < G;
  const int Hq = p.num_q_heads;
  // Chunks per split and this unit's splits: fixed by the launch, or, for a
  // ragged batch, item blockIdx.x of the work list the selection wrote (the
  // 1-D grid's workgroups past the list leave here).
  int cps = p.cps, S = p.splits;
  if (kPlan) {
    const int w = blockIdx.x;
    const int items = p.plan[0];
    cps = min(max(p.plan[1], 1), kMaxSplitChunks);
    const uint32_t e = (uint32_t)p.plan[kPlanHeader + w];   // the grid never exceeds the list's room
    if (w >= items) return;
    plan_unpack(e, q, g, s, S);
    q = min(q, p.num_q - 1);
    g = min(g, Hkv - 1);
    S = min(max(S, 1), p.splits);
    s = min(s, S - 1);
  }
  const int32_t* prow = p.pos + (int64_t)q * p.width;
  const int c0 = s * cps;                   // first chunk of this workgroup's split
  const int cfirst = c0 + wave;

  // Prologue: the block heads of the split go to LDS, the query rows to
  // registers, with the valid length and the first slot; every load is
  // issued before any is waited for (one memory round trip).
  for (int h = tid; h < 8 * cps; h += kAttnThreads) {
    const int run = 8 * c0 + h;
    const int i = p.run_heads ? run : 4 * run;
    heads_s[h] = i < p.width ? prow[i] : 0;
  }
  const int npos_given = p.n_pos[q];
  // never past the buffer (a row of run heads covers 4 positions an entry)
  const int npos = min(max(npos_given, 0), p.run_heads ? 4 * p.width : p.width);
  const int slot0 = max(prow[0], 0);       // masked loads read here (a row without positions holds -1)
#ifdef QSA_DEBUG_CHECKS
  // the run rule over this workgroup's positions, and the length
  if (!p.run_heads) {
    if (tid == 0 && s == 0 && g == 0)
      QSA_DCHECK(p.err, npos_given >= 1 && npos_given <= p.width, QSA_ERROR_BAD_POSITIONS);
    for (int i = 32 * c0 + tid; i < min(32 * (c0 + cps), min(npos, p.width)); i += kAttnThreads)
      QSA_DCHECK(p.err, prow[i] == prow[i & ~3] + (i & 3), QSA_ERROR_BAD_POSITIONS);
  }
#endif
  bf16x8 qb[4];
  {
    const uint16_t* qrow = p.q + ((int64_t)q * Hq + g * G + j) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = hvalid ? *reinterpret_cast<const u32x4*>(qrow + kdim<kFp8>(kk, kg)) : u32x4{0u, 0u, 0u, 0u};
      qb[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float kscale = kFp8 ? p.k_scale[g] : 1.f;
  const float vscale = kFp8 ? p.v_scale[g] : 1.f;
  const float sl2 = p.sm_scale_log2 * kscale;
  const uint32_t row_stride = (uint32_t)(Hkv * D * EB);   // bytes between consecutive slots
  const uint8_t* kbase = p.kc + (int64_t)g * D * EB;
  const uint8_t* vbase = p.vc + (int64_t)g * D * EB;
  const int nchunks = (npos + kChunk - 1) / kChunk;
  const int c_end = min(c0 + cps, nchunks);
  // a work list sized the unit's splits from the metadata; the selection's
  // count must fit them
  if (kPlan && tid == 0 && s == 0) QSA_DCHECK(p.err, nchunks <= S * cps, QSA_ERROR_BAD_POSITIONS);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Main loop.  With kKL (the non-temporal, large-batch kernels) a chunk's K
  // rows go to the wave's LDS buffer through direct-to-LDS loads of whole
  // lines and its V rows to registers; otherwise both go to registers.
  // FP8: two chunk buffers in ping-pong, the next chunk's loads are in flight
  // while this chunk is computed (with kKL an issue is always KL::kLoads + 8
  // vector-memory operations, so waiting for that many to remain outstanding
  // means the current chunk has landed; the compiler does not track the LDS
  // the loads write, so these waits are explicit).  BF16 (twice the bytes per
  // chunk) keeps one chunk per wave in flight and relies on more waves.
  constexpr bool kKL = kNt;
  uint8_t* kbuf0 = kbuf_a[wave];
  if (kFp8) {
    // sched_barrier keeps the compiler from sinking a chunk's loads down to
    // its compute (which would serialise load latency and math again).
    uint8_t* kbuf1 = kbuf_b[wave];
    constexpr int kIssueOps = KL::kLoads + 8;
    ChunkRaw<kFp8, kKL> ca, cb;
    const int nl = cfirst < c_end ? npos : 0;
    issue_chunk<kFp8, kNt, kKL>(ca, kbuf0, lds_heads<kFp8, kKL>(heads_s, cfirst - c0, cps, lane, j, kg),
                                cfirst * kChunk, nl, slot0, kbase, vbase, row_stride, lane, j, kg);
    __builtin_amdgcn_sched_barrier(0);
    for (int c = cfirst; c < c_end; c += 2 * kAttnWaves) {
      const int cn = c + kAttnWaves;
      issue_chunk<kFp8, kNt, kKL>(cb, kbuf1, lds_heads<kFp8, kKL>(heads_s, cn - c0, cps, lane, j, kg),
                                  cn * kChunk, cn < c_end ? npos : 0, slot0, kbase, vbase, row_stride, lane, j, kg);
      __builtin_amdgcn_sched_barrier(0);
      if (kKL) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kIssueOps));
      compute_chunk<kFp8, kKL>(ca, kbuf0, qb, sl2, m_run, l_run, o, j, kg);
      if (kKL) __builtin_amdgcn_s_waitcnt(kWaitLds);       // buffer 0 read out before it is refilled
      __builtin_amdgcn_sched_barrier(0);
      if (cn >= c_end) break;
      const int cnn = cn + kAttnWaves;
      issue_chunk<kFp8, kNt, kKL>(ca, kbuf0, lds_heads<kFp8, kKL>(heads_s, cnn - c0, cps, lane, j, kg),
                                  cnn * kChunk, cnn < c_end ? npos : 0, slot0, kbase, vbase, row_stride, lane, j,
                                  kg);
      __builtin_amdgcn_sched_barrier(0);
      if (kKL) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kIssueOps));
      compute_chunk<kFp8, kKL>(cb, kbuf1, qb, sl2, m_run, l_run, o, j, kg);
      if (kKL) __builtin_amdgcn_s_waitcnt(kWaitLds);       // buffer 1 read out before it is refilled
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int c = cfirst; c < c_end; c += kAttnWaves) {
      ChunkRaw<kFp8, kKL> cur;
      issue_chunk<kFp8, kNt, kKL>(cur, kbuf0, lds_heads<kFp8, kKL>(heads_s, c - c0, cps, lane, j, kg), c * kChunk,
                                  npos, slot0, kbase, vbase, row_stride, lane, j, kg);
      if (kKL) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      compute_chunk<kFp8, kKL>(cur, kbuf0, qb, sl2, m_run, l_run, o, j, kg);
      if (kKL) __builtin_amdgcn_s_waitcnt(kWaitLds);
    }
  }
  // The last prefetch of a FP8 wave (a masked chunk past the end) may still
  // be writing LDS: drain it before the workgroup can finish.
  if (kKL) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // Row sums over the 4 lane groups of a head.
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  // Lane (kg, j) holds O[head j][32kg + 8rr + u] = o[u][rr].
  if (hvalid) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float* dst = &o_s[wave][j][32 * kg + 8 * rr];
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[0][rr], o[1][rr], o[2][rr], o[3][rr]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4][rr], o[5][rr], o[6][rr], o[7][rr]};
    }
    if (kg == 0) {
      m_s[wave][j] = m_run;
      l_s[wave][j] = l_run;
    }
  }
  __syncthreads();

  const int nout = G * D;
  if (S == 1) {
    // 4 consecutive outputs of one head per thread
    for (int v4 = tid; v4 < nout / 4; v4 += kAttnThreads) {
      const int hh = (4 * v4) / D, d = (4 * v4) % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
      f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float sc = m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M);
        num += sc * *reinterpret_cast<const f32x4*>(&o_s[w][hh][d]);
        den += sc * l_s[w][hh];
      }
      num *= vscale / den;
      store_out<kOutBf16>(p.out, ((int64_t)q * Hq + g * G) * D + 4 * v4, num);
    }
    return;
  }

  // Split partial: [G*128 unnormalised O][16 m][16 l] floats per (q, g, s),
  // written with 16-byte device-scope stores (they bypass the per-XCD caches),
  // so no cache flush is needed before the arrival is counted; only the
  // stores' completion.
  const int pstride = G * D + 32;
  float* unit = p.part + ((int64_t)q * Hkv + g) * p.splits * pstride;
  const __amdgpu_buffer_rsrc_t unit_rs = partial_rsrc(unit);
  const int mine = s * pstride;
  for (int v4 = tid; v4 < nout / 4; v4 += kAttnThreads) {
    const int hh = (4 * v4) / D, d = (4 * v4) % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
    f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float sc = m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M);
      val += sc * *reinterpret_cast<const f32x4*>(&o_s[w][hh][d]);
    }
    store_coherent(unit_rs, mine + 4 * v4, val);
  }
  // m (heads 0..15) then l (heads 0..15): one value per thread
  if (tid < 32) {
    const int hh = tid & 15;
    float M = -INFINITY, den = 0.f;
    if (hh < G) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w)
        den += (m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M)) * l_s[w][hh];
    }
    store_coherent_f32(unit_rs, mine + nout + tid, tid < 16 ? M : den);
  }
  __builtin_amdgcn_s_waitcnt(0);     // this thread's stores have reached the coherence point
  __syncthreads();
  uint32_t* const ctr = p.counters + (q * Hkv + g) * kCounterStride;
  if (tid == 0) {
    const uint32_t ticket = atomicAdd(ctr, 1u);
    s_last = ticket == (uint32_t)(S - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Last workgroup of the unit: device-scope loads bring, straight into
  // registers, every split's numerators of each thread's 4 outputs (one
  // round for groups of <= 8 heads; splits past S re-read the last one and
  // are not weighed).  The 32 lanes of a wave half share one head (128
  // outputs): lane t of the half loads split t's maximum and sum of that
  // head, the half reduces them, and each lane reads the split weights from
  // the lanes that hold them.
  const bool upper = lane >= 32;
  const int tl = lane & 31;
  static_assert(kMaxSplits <= 32, "one split per lane of a wave half");
  for (int v0 = 0; v0 < nout / 4; v0 += kAttnThreads) {
    const int v4 = min(v0 + tid, nout / 4 - 1);
    const int hh = (4 * v4) / D;
    f32x4 vals[kMaxSplits];
#pragma unroll
    for (int t = 0; t < kMaxSplits; ++t) vals[t] = load_coherent(unit_rs, min(t, S - 1) * pstride + 4 * v4);
    const int ts = min(tl, S - 1) * pstride + nout + hh;
    const float m_own = load_coherent_f32(unit_rs, ts);
    const float l_own = load_coherent_f32(unit_rs, ts + 16);
    const float mv = tl < S ? m_own : -INFINITY;
    const float M = half32_max(mv);
    const float w_own = mv == -INFINITY ? 0.f : exp2f(mv - M);
    const float den = half32_sum(tl < S ? w_own * l_own : 0.f);
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kMaxSplits; ++t) {
      if (t < S) {
        const float w_lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_own), t));
        const float w_hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_own), 32 + t));
        num += (upper ? w_hi : w_lo) * vals[t];
      }
    }
    if (v0 + tid < nout / 4) {
      num *= vscale / den;
      store_out<kOutBf16>(p.out, ((int64_t)q * Hq + g * G) * D + 4 * v4, num);
    }
  }
  if (tid == 0) ctr[0] = 0u;
}

size_t attn_plan_bytes(int num_q, int num_kv_heads, int width) {
  if (num_q * num_kv_heads >= kAttnTargetWgs) return 0;
  const AttnSplit sp = attn_split(num_q, num_kv_heads, width, true);
  return (size_t)(kPlanHeader + (int64_t)num_q * num_kv_heads * sp.splits) * sizeof(int32_t);
}

size_t attn_partial_bytes(int num_q, int num_kv_heads, int group, int width) {
  // sized for the ragged geometry whenever a batch could take it (it has at
  // least the splits of the uniform one)
  const AttnSplit sp = attn_split(num_q, num_kv_heads, width, num_q * num_kv_heads < kAttnTargetWgs);
  if (sp.splits <= 1) return 0;
  return (size_t)num_q * num_kv_heads * sp.splits * (group * QSA_HEAD_DIM + 32) * sizeof(float);
}

hipError_t launch_attn(const Meta& m, const AttnArgs& a, hipStream_t stream) {
  // the split geometry follows the positions (4 per run head)
  const int pos_width = a.run_heads ? QSA_BLOCK * (a.width - 1) + QSA_BLOCK - 1 : a.width;
  // the ragged geometry only with a work list (qsa_decode on a ragged batch)
  const bool ragged = a.plan != nullptr && attn_ragged(m.num_req, m.num_q, a.num_kv_heads);
  const AttnSplit sp = attn_split(m.num_q, a.num_kv_heads, pos_width, ragged);
  AttnParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kc = static_cast<const uint8_t*>(a.k_cache);
  p.vc = static_cast<const uint8_t*>(a.v_cache);
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.pos = a.pos;
  p.n_pos = a.n_pos;
  p.out = a.out;
  p.part = a.partials;
  p.counters = a.counters;
  p.width = a.width;
  p.run_heads = a.run_heads;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.sm_scale_log2 = a.sm_scale * 1.4426950408889634f;
  p.splits = sp.splits;
  p.cps = sp.chunks_per_split;
  p.err = a.err;
  p.plan = ragged ? a.plan : nullptr;
  p.num_q = m.num_q;
  // a ragged batch with a work list: one workgroup per item, as many as the
  // list can hold (those past its length leave at once)
  const dim3 grid = p.plan != nullptr ? dim3((unsigned)(m.num_q * a.num_kv_heads * sp.splits))
                                      : dim3((unsigned)m.num_q, (unsigned)a.num_kv_heads, (unsigned)sp.splits);
  // Large batches stream K/V with non-temporal loads (measured faster once
  // the (query, KV head) units alone fill the chip); small ones keep the
  // default policy (faster there).
  const bool nt = (int64_t)m.num_q * a.num_kv_heads >= kNtMinUnits;
#define QSA_ATTN_LAUNCH(F8, OB)                                                       \
  do {                                                                                 \
    if (p.plan && nt) attn_kernel<F8, OB, true, true><<<grid, kAttnThreads, 0, stream>>>(p);   \
    else if (p.plan) attn_kernel<F8, OB, false, true><<<grid, kAttnThreads, 0, stream>>>(p);  \
    else if (nt) attn_kernel<F8, OB, true><<<grid, kAttnThreads, 0, stream>>>(p);              \
    else attn_kernel<F8, OB, false><<<grid, kAttnThreads, 0, stream>>>(p);                     \
  } while (0)
  if (a.kv_fp8) {
    if (a.out_bf16) QSA_ATTN_LAUNCH(true, true);
    else QSA_ATTN_LAUNCH(true, false);
  } else {
    if (a.out_bf16) QSA_ATTN_LAUNCH(false, true);
    else QSA_ATTN_LAUNCH(false, false);
  }
#undef QSA_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace qsa
