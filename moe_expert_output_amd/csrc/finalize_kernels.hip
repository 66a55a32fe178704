// finalize_kernels.hip -- gfx950 kernels and C ABI of the MoE finalize library.
//
// Sources (cited by key):
//   [FI6631]  flashinfer PR #6631, "perf(comm): gather MoE-finalize routes together and accumulate
//             in FP32": Description (indices and scales of the routes loaded before their rows,
//             float32 accumulation rounded once, residual add + RMSNorm on the rounded sum),
//             test changes (-1 routes, top_k 6/8/10, swizzled scale buffer size).
//   [TR16778] TensorRT-LLM PR #16778, "MoE: fp32 accumulation in deferred MoEAllReduce finalize":
//             Fix (top-k sum and shared add in a float32 array, rounded once).
//   [FI6546]  flashinfer PR #6546, small-batch trtllm-gen finalize: Description (one block per
//             token and hidden slice, 128-bit loads, top-k split over thread groups combined in
//             shared memory, top_k <= 64).
//   [FI3385]  flashinfer PR #3385, "feat: MNNVL Allreduce quant fusion and performance
//             optimization": walkthrough (FP8 / NVFP4 outputs, SF layouts), review comments
//             (vector-width guard, layout whitelist, null-guarded optional outputs).
//
// Kernel design (gfx950, wave64). One workgroup handles one token and a contiguous range of
// 8-element (16-byte) hidden slots. For the RMSNorm modes the range is the whole row, or, with a
// caller's workspace, one of S slices of it whose partial sums of squares are exchanged through
// that workspace (see "Split rows"). The workgroup's lanes are split into G route groups of
// L lanes (L a multiple of 64, so every wavefront belongs to one group); group g takes routes
// g, g+G, g+2G, ... Every wavefront first loads all K indices and scales of its token in one
// coalesced load (lane k holds route k) and reads them back with readlane, so row addresses are
// wave-uniform; it then issues every present route's 128-bit row load (in chunks of at most 16
// routes) before it consumes any of them, accumulates in float32, and hands its partials to group 0
// through LDS, which adds them in group order (deterministic). Group 0 applies the routed
// scaling and shared add, rounds once, adds the residual, and reduces the sum of squares with a
// DPP wavefront reduction plus one LDS pass across wavefronts. Quantized outputs are encoded
// with gfx950's FP4/FP8 conversion instructions, made exact (the code of the exact product or
// quotient, ties included) by the steps described at the encoders in device_utils.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <initializer_list>

#include "../../include/moe_finalize.h"
#include "device_utils.h"

namespace mfin {

enum : int { MODE_FIN = 0, MODE_RMS = 1, MODE_NVFP4 = 2, MODE_FP8 = 3 };

struct Params {
  // The launch shape and what the first loads address, together at the front so that they
  // arrive in one batch of scalar loads (see the start of finalize_kernel).
  int T, H, K;
  int slices;                // workgroups per token (> 1: the row is split, see below)
  int xcd_map;               // split rows: a token's slices share one XCD (see the kernel)
  int main_blocks;           // workgroups before the scale-padding ones
  int route_stride;          // > 0: no route map; route k of token t is row k * route_stride + t
  int scales_bf16;
  int nv;                    // H / 8 slots per row
  int lanes;                 // L: lanes per route group (multiple of 64)
  int slot_span;             // slots covered by one workgroup (L * P)
  int pad_blocks;            // NVFP4, swizzled scales: workgroups after the token ones that
                             // only zero the scale bytes of the padding rows
  uint32_t slice_magic;      // ceil(2^32 / slices) where q * slices < 2^32 for every workgroup
                             // index q, so q / slices = mulhi(q, slice_magic); else 0
  const int32_t* idx;        // [T, K]
  const void* scales;        // [T, K] fp32 or bf16, or null
  const uint8_t* shared;     // [T, H] or null
  const uint8_t* residual;   // [T, H]
  const uint8_t* gamma;      // [H]
  uint8_t* ws;               // workspace of the split row modes (null when slices == 1)
  const uint8_t* rows;       // [n_rows, H] act dtype
  int64_t n_rows;
  float rsf;
  float eps;
  float inv_h;
  int sf_swizzled;
  uint8_t* out;              // MODE_FIN: finalize output; else norm_out (nullable in quant)
  uint8_t* residual_out;     // nullable
  uint8_t* quant_out;
  uint8_t* sf_out;
  const float* qscale;
  uint32_t spin_limit;       // split rows: polls of a slice's word before the wait gives up
  int split_quant;           // quantized outputs: route group 1 encodes half of the codes
};

// Split rows. When a token's row is spread over `slices` workgroups, each workgroup publishes
// the sum of squares of its slice in the caller's workspace and waits for the other slices of
// its token. Layout: a 256-byte header whose first word is a sticky timeout flag, then one
// 128-byte block (one cache line) per token holding kMaxSlices 64-bit slots. A slot carries
// (epoch << 32 | float bits of a partial) in ONE relaxed device-scope atomic word, so the flag and
// the data become visible together and no release/acquire fences (L2 writeback / invalidate) are
// needed. All kMaxSlices slots of a token hold the same epoch between calls: slice j rewrites
// every slot m with m % slices == j (its own slot j carries its partial), so a call reads the
// current epoch from its own slot and waits until slots 0..slices-1 carry epoch + 1. Only slice j
// writes the slots m == j (mod slices), so a slice that starts late still reads the old epoch,
// finds the others' new one and completes, leaving every slot on the new epoch. A zero-filled
// workspace is valid, no call needs a reset (also after a timeout), and the slice count may
// change from call to call. When a slice gives up waiting (spin_limit polls), it sets the header
// flag and counts the missing partials as NaN, so its part of norm_out (and of the quantized
// outputs) is NaN rather than a wrong finite value; residual_out is unaffected.
constexpr int kMaxSlices = 16;
constexpr size_t kWsHeader = 256, kWsPerToken = 8 * kMaxSlices;
constexpr uint32_t kMaxSpins = 1u << 22;      // ~0.1-0.5 s of polling, then give up (flagged)
constexpr uint32_t kQuietNaN = 0x7FC00000u;

// Raw buffer resource over `bytes` bytes at `base` (gfx9-family descriptor word 3: 32-bit data
// format, no swizzle). Loads outside [0, bytes) return zeros and stores there are dropped, so an
// absent route, a missing optional tensor or a lane past the row needs no branch: its buffer is
// empty or its offset is out of range.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Partial sums of route groups g >= 1: [G-1][P][L] x 8 floats.
extern __shared__ float4 lds_dyn[];

// Where quantized outputs go (shared by the fused epilogue and the standalone quantizer).
struct QuantDst {
  uint8_t* sf_out;    // NVFP4 block scales
  int H;
  int sf_swizzled;
};

// Quantize the 8 rounded values `nr` of slot `s` of row `t` (this lane) and store the codes
// through `q_r` (the row's code buffer); for NVFP4 also the block scales. Every lane of the
// wavefront must call it (the NVFP4 block amax and scale gathers are cross-lane). Lanes with
// live == false hold zeros and store nothing.
// NTQ: the aux bits of the FP8 code stores (the fused kernel passes its nontemporal choice:
// same-box A/B, cold, FP8 at T = 64 / 128 / 512: 0.18 / 0.35 / 0.58 us faster; the NVFP4 code
// stores, 4 bytes per lane, stay cacheable: nontemporal was 0.37 us slower at T = 512).
// HALF (NVFP4 only): 0 encodes all 8 elements; 1 only elements 0..3 (and the block scales),
// 2 only elements 4..7, for two wavefronts that share one lane's values (each needs all 8 for
// the block amax).
template <int MODE, int NTQ = 0, int HALF = 0>
__device__ __forceinline__ void quantize_store(const float nr[8], double qs,
                                               const __amdgpu_buffer_rsrc_t& q_r, uint32_t voff,
                                               bool live, int s, int t, const QuantDst& d) {
  static_assert(HALF == 0 || MODE == MODE_NVFP4, "only the NVFP4 codes are split");
  constexpr int E0 = HALF == 2 ? 4 : 0, E1 = HALF == 1 ? 4 : 8;
  if constexpr (MODE == MODE_FP8) {
    const u32x2 q = e4m3_pack8_exact(nr, (float)qs);   // exact: the caller's float32 scale
    __builtin_amdgcn_raw_buffer_store_b64(q, q_r, voff >> 1, 0, NTQ);
  } else {
    // NVFP4: a 16-element block is this lane's 8 elements and the neighbouring lane's 8.
    // A NaN anywhere in the block makes its amax NaN: scale code 0x7F and all-zero codes.
    // Magnitude bit patterns order like the magnitudes, with NaN above infinity, so one
    // unsigned maximum gives both the block amax and the NaN test.
    uint32_t amax_bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      amax_bits = max(amax_bits, __builtin_bit_cast(uint32_t, nr[e]) & 0x7FFFFFFFu);
    amax_bits = pair_max_u32(amax_bits);
    const bool nan_blk = amax_bits > 0x7F800000u;
    const float amax = __builtin_bit_cast(float, amax_bits);
    const float gs = (float)qs;                 // exact: the caller's float32 scale
    uint32_t sfc, word = 0;
    if (gs >= 0x1p-100f && gs <= 0x1p100f) {
      // the branch-free exact encoders for the usual range of global scales (a uniform
      // branch: gs is the same for every lane)
      sfc = nan_blk ? 0x7Fu : e4m3_block_scale_exact(amax, gs);
      word = e2m1_pack_exact<E1 - E0>(nr + E0, gs, e4m3_value_hw(sfc));
    } else {
      // beyond it, float64 for the block scale and per-midpoint tests for the codes
      sfc = nan_blk ? 0x7Fu : e4m3_code((double)amax * qs / 6.0);
      const float sf = (float)e4m3_value(sfc);  // exact: an E4M3 value
      // a zero block scale gives signed zero codes (a NaN block is cleared below)
      const uint32_t keep = sfc != 0 ? 7u : 0u;
#pragma unroll
      for (int e = E0; e < E1; ++e) {
        const uint32_t m = e2m1_code(__builtin_fabsf(nr[e]), gs, sf) & keep;
        word |= (m | (sign_bit(nr[e]) << 3)) << (4 * (e - E0));
      }
    }
    word = nan_blk ? 0u : word;
    if constexpr (HALF == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(word, q_r, voff >> 2, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)word, q_r,
                                            (voff >> 2) + (HALF == 2 ? 2u : 0u), 0, 0);
      if constexpr (HALF == 2) return;         // the block scales come from the other half
    }
    // Scale bytes: lanes 8m..8m+7 hold blocks 4m'..4m'+3 (two lanes per block).
    const uint32_t sf_here = live ? sfc : 0u;
    // (a workgroup's slot span is a multiple of 8, so the storing lanes are lanes 8m and read
    // lanes 8m + 2, 4, 6 of their own 16-lane row)
    const uint32_t b1 = row_shl_dpp<2>(sf_here);
    const uint32_t b2 = row_shl_dpp<4>(sf_here);
    const uint32_t b3 = row_shl_dpp<6>(sf_here);
    if (live && (s & 7) == 0) {
      const int b = s >> 1;                      // first block of the group of four
      const int nb = d.H >> 4;
      const uint32_t packed = sf_here | (b1 << 8) | (b2 << 16) | (b3 << 24);
      if (d.sf_swizzled) {
        const int nb4 = (nb + 3) & ~3;
        const int64_t off = ((int64_t)(t >> 7) * (nb4 >> 2) + (b >> 2)) * 512 + (t & 31) * 16 +
                            ((t & 127) >> 5) * 4;
        *(uint32_t*)(d.sf_out + off) = packed;   // padding blocks carry sf 0
      } else {
        uint8_t* dst = d.sf_out + (int64_t)t * nb + b;
        const uint8_t bytes[4] = {(uint8_t)sf_here, (uint8_t)b1, (uint8_t)b2, (uint8_t)b3};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (b + i < nb) dst[i] = bytes[i];
      }
    }
  }
}

// Zero the swizzled scale bytes of the padding rows (T up to the next multiple of 128). Only the
// last 128-row tile has padding rows. Row r's word of a 512-byte tile sits at byte
// (r % 32) * 16 + (r / 32) * 4, so word w of a tile belongs to row (w / 4) + 32 * (w % 4). The
// tile's words are split over every thread of the grid (`thread` of `n_threads`) in grid-stride
// order, so each wavefront store covers consecutive words; the words of rows below T hold
// other workgroups' scales and are skipped.
__device__ __forceinline__ void zero_sf_padding(const QuantDst& d, int T, int64_t thread,
                                                int64_t n_threads) {
  const int rem = T & 127;
  if (rem == 0) return;
  const int tiles = (((d.H >> 4) + 3) & ~3) >> 2;
  uint8_t* const last = d.sf_out + (int64_t)(T >> 7) * tiles * 512;
  const int n_words = tiles * 128;
  for (int64_t w = thread; w < n_words; w += n_threads) {
    const int within = (int)(w & 127);
    const int row = (within >> 2) + 32 * (within & 3);
    if (row >= rem) *(uint32_t*)(last + (int64_t)(w >> 7) * 512 + within * 4) = 0u;
  }
}

// NT = 2 marks the streamed accesses nontemporal (chosen for large calls): the row, shared and
// residual loads, the residual_out and norm_out stores and the FP8 code stores; gamma, shared by
// every token, stays cacheable. NT = 0 leaves them all cacheable.
template <int ACT, int MODE, int G, int P, int JMAX, int NT>
__global__ __launch_bounds__(1024) void finalize_kernel(const Params a) {
  // blockIdx.x = token * slices + slice (one slice per token in the whole-row modes). For NVFP4
  // with swizzled scales, pad_blocks workgroups after those only zero the scale bytes of the
  // padding rows (same-box A/B: after the token workgroups beat before them by up to 0.2 us at
  // T = 64, and beat zeroing in the token workgroups, which cost 1 us at T = 1 when few of
  // their wavefronts are idle). They wait on nothing, so no split row's exchange waits on them.
  // The fields the prologue branches on or builds addresses from, fetched in one batch: left
  // to itself the compiler loads each field at its first use, so every early branch (padding
  // workgroups, XCD map, tokens past T) waited for a scalar load of its own, a chain of
  // dependent round trips before the first vector load. The last field brings the struct's
  // last 64-byte line into the scalar cache with the others, so the epilogue's loads of the
  // remaining fields hit there.
  asm volatile("" ::"s"(a.T), "s"(a.H), "s"(a.K), "s"(a.slices), "s"(a.xcd_map),
               "s"(a.main_blocks), "s"(a.route_stride), "s"(a.scales_bf16), "s"(a.nv),
               "s"(a.lanes), "s"(a.slot_span), "s"(a.slice_magic), "s"(a.idx), "s"(a.scales),
               "s"(a.shared), "s"(a.residual), "s"(a.gamma), "s"(a.ws), "s"(a.split_quant));
  const int bid = blockIdx.x;
  if constexpr (MODE == MODE_NVFP4) {
    const int n_main = a.main_blocks;
    if (bid >= n_main) {
      zero_sf_padding(QuantDst{a.sf_out, a.H, 1}, a.T,
                      (int64_t)(bid - n_main) * blockDim.x + threadIdx.x,
                      (int64_t)a.pad_blocks * blockDim.x);
      return;
    }
  }
  // Workgroup -> (token, slice). Workgroup b runs on XCD b % 8, so with a.xcd_map the slices of
  // token t are the workgroups (g * slices + j) * 8 + t % 8 (g = t / 8): all on one XCD, where
  // they start together, instead of on consecutive XCDs, whose start times differ by up to
  // ~0.5 us that the exchange would wait for (the host's xcd_mapped chooses when). Workgroups
  // of tokens past T (T not a multiple of 8) exit at once.
  // q / slices: one scalar multiply-high where the host found the reciprocal exact, instead of
  // an integer division (a float reciprocal and some forty instructions before the first load).
  const auto div_slices = [&](int q) -> int {
    if (a.slices == 1) return q;
    return a.slice_magic ? (int)__umulhi((uint32_t)q, a.slice_magic) : q / a.slices;
  };
  int t, slice;
  if (a.xcd_map) {
    const int q = bid >> 3;
    const int grp = div_slices(q);
    slice = q - grp * a.slices;
    t = (grp << 3) + (bid & 7);
    if (t >= a.T) return;
  } else {
    t = div_slices(bid);
    slice = bid - t * a.slices;
  }
  const int tid = threadIdx.x;
  const int L = a.lanes;
  // Wave-uniform route group. Groups are whole wavefronts, so scalar compares of the wavefront
  // index replace a per-lane integer division that stood before the first load.
  int g = 0;
  if constexpr (G > 1) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lw = L >> 6;
    g = (wave >= lw) + (G > 2 ? (wave >= 2 * lw) + (wave >= 3 * lw) : 0);
  }
  const int lane = tid - g * L;
  const int slot0 = slice * a.slot_span;
  const uint32_t row_bytes = (uint32_t)a.H * 2;
  const int64_t tok_off = (int64_t)t * row_bytes;

  // Byte offset of each of this lane's 16-byte slots in a row. Lanes past the row or past this
  // workgroup's slice get an out-of-range offset: their buffer loads read zeros and their
  // buffer stores are dropped, so no branch guards any memory access.
  uint32_t voff[P];
  bool live[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int sl = slot0 + lane + p * L;
    live[p] = sl < a.nv && (lane + p * L) < a.slot_span;
    voff[p] = live[p] ? (uint32_t)sl * 16u : kOutOfRange;
  }

  // ---- route metadata: all K indices and scales of the token, one coalesced load per
  // wavefront (lane k holds route k), issued before any row load; read back with readlane so
  // every row address is wave-uniform.
  const int lane64 = tid & 63;
  const bool bf16_scales = a.scales_bf16 != 0;
  const uint32_t my_idx = __builtin_amdgcn_raw_buffer_load_b32(
      rsrc(a.idx + (int64_t)t * a.K, a.route_stride ? 0u : (uint32_t)a.K * 4u),
      (uint32_t)lane64 * 4u, 0, 0);
  // Raw scale bits of both formats; the unused (or missing) one has an empty buffer. Loads are
  // predicated by buffer size, never by branches: a branch join makes the compiler wait for
  // every outstanding load before the row loads are issued.
  const uint32_t my_w32 = __builtin_amdgcn_raw_buffer_load_b32(
      rsrc((const uint8_t*)a.scales + (int64_t)t * a.K * 4,
           (a.scales && !bf16_scales) ? (uint32_t)a.K * 4u : 0u),
      (uint32_t)lane64 * 4u, 0, 0);
  const uint32_t my_w16 = __builtin_amdgcn_raw_buffer_load_b16(
      rsrc((const uint8_t*)a.scales + (int64_t)t * a.K * 2,
           (a.scales && bf16_scales) ? (uint32_t)a.K * 2u : 0u),
      (uint32_t)lane64 * 2u, 0, 0);
  [[maybe_unused]] double qs = 0.0;
  if constexpr (MODE == MODE_NVFP4 || MODE == MODE_FP8) qs = (double)*a.qscale;
  // Split rows: this slice's current epoch (the upper half of its exchange word), read now so the
  // barrier does not wait for it. Every wavefront reads it unconditionally (from gamma, a valid
  // dummy, when rows are whole): a load under a branch would make the compiler wait for it at the
  // branch join. Only the 32 bits in use are loaded: with a 64-bit load the compiler reused the
  // unused half's register at once, and that wait held the first row load back until this
  // memory-side load had returned.
  [[maybe_unused]] uint32_t epoch_prev = 0;
  if constexpr (MODE != MODE_FIN) {
    const uint32_t* ep =
        a.slices > 1
            ? (const uint32_t*)((const uint64_t*)(a.ws + kWsHeader + (size_t)t * kWsPerToken) +
                                slice) + 1
            : (const uint32_t*)a.gamma;
    epoch_prev = __hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Group 0 also needs the shared-expert, residual and gamma slices; issue them alongside.
  u32x4 shv[P], resv[P], gamv[P];
  {
    const auto sh_r = rsrc(a.shared + tok_off, (g == 0 && a.shared) ? row_bytes : 0u);
#pragma unroll
    for (int p = 0; p < P; ++p) shv[p] = __builtin_amdgcn_raw_buffer_load_b128(sh_r, voff[p], 0, NT);
    if constexpr (MODE != MODE_FIN) {
      const auto res_r = rsrc(a.residual + tok_off, g == 0 ? row_bytes : 0u);
      const auto gam_r = rsrc(a.gamma, g == 0 ? row_bytes : 0u);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        resv[p] = __builtin_amdgcn_raw_buffer_load_b128(res_r, voff[p], 0, NT);
        gamv[p] = __builtin_amdgcn_raw_buffer_load_b128(gam_r, voff[p], 0, 0);
      }
    }
  }

  // ---- row gather: per chunk of CH routes, issue every route's 128-bit loads (an absent
  // route's buffer is empty and reads zeros), then accumulate the present ones in float32 ----
  // exactly one of the two scale buffers is non-empty, the other reads zeros
  const uint32_t my_wbits = my_w32 | (my_w16 << 16);
  // Rank sums (route_stride != 0) have an empty index buffer, which reads 0, and take row
  // kk * route_stride + t: one formula for both, with no branch between the row loads.
  const int t_rs = a.route_stride ? t : 0;
  constexpr int CH = JMAX < 16 / P ? JMAX : 16 / P;
  float acc[P][8];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[p][e] = 0.f;
#pragma unroll
  for (int c0 = 0; c0 < JMAX; c0 += CH) {
    if (g + c0 * G >= a.K) break;
    float w[CH];
    bool present[CH];
    u32x4 v[CH][P];
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
      const int k = g + (c0 + jj) * G;
      const int kk = k < a.K ? k : 0;
      const int pidx = __builtin_amdgcn_readlane((int)my_idx, kk) + kk * a.route_stride + t_rs;
      present[jj] = k < a.K && (uint32_t)pidx < (uint32_t)a.n_rows;
      const uint32_t wbits = (uint32_t)__builtin_amdgcn_readlane((int)my_wbits, kk);
      // an absent route's scale is never used: its weight is 0 (and its row reads zeros)
      w[jj] = present[jj] ? (a.scales ? __builtin_bit_cast(float, wbits) : 1.f) : 0.f;
      // an absent route gets an empty buffer: its loads read zeros and touch no memory
      const auto row_r = rsrc(a.rows + (int64_t)pidx * row_bytes, present[jj] ? row_bytes : 0u);
#pragma unroll
      for (int p = 0; p < P; ++p) v[jj][p] = __builtin_amdgcn_raw_buffer_load_b128(row_r, voff[p], 0, NT);
    }
    // Every row load of the chunk is issued before the first use: without this barrier the
    // scheduler may unpack an early route (and wait for it) between the later routes' loads.
    __builtin_amdgcn_sched_barrier(0);
    // Every route is accumulated (an absent one adds 0 * 0): a use under a branch would let the
    // compiler sink the load into it and serialize the row loads.
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float x[8];
        Act<ACT>::unpack(v[jj][p], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[p][e] = __builtin_fmaf(w[jj], x[e], acc[p][e]);
      }
      // with 16 loads in a chunk, accumulate route by route so the unpacked values of later
      // routes do not pile up in registers (that spilled)
      if constexpr (CH * P > 8) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- combine the route groups through LDS, in group order ----
  if constexpr (G > 1) {
    if (g > 0) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float4* dst = lds_dyn + ((size_t)((g - 1) * P + p) * L + lane) * 2;
        dst[0] = make_float4(acc[p][0], acc[p][1], acc[p][2], acc[p][3]);
        dst[1] = make_float4(acc[p][4], acc[p][5], acc[p][6], acc[p][7]);
      }
    }
    lds_barrier();
    if (g == 0) {
      // every group's partials are read first (the reads overlap), then added in group order
      float4 u[G - 1][P][2];
#pragma unroll
      for (int gg = 1; gg < G; ++gg)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float4* src = lds_dyn + ((size_t)((gg - 1) * P + p) * L + lane) * 2;
          u[gg - 1][p][0] = src[0];
          u[gg - 1][p][1] = src[1];
        }
#pragma unroll
      for (int gg = 1; gg < G; ++gg) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float4 u0 = u[gg - 1][p][0], u1 = u[gg - 1][p][1];
          acc[p][0] += u0.x; acc[p][1] += u0.y; acc[p][2] += u0.z; acc[p][3] += u0.w;
          acc[p][4] += u1.x; acc[p][5] += u1.y; acc[p][6] += u1.z; acc[p][7] += u1.w;
        }
      }
    }
  }

  // ---- routed scaling, shared add, the one rounding; then residual add ----
  float r[P][8];
  u32x4 r_pk[P];
  float ss = 0.f;
  if (g == 0) {
    const auto fin_r = rsrc(a.out + tok_off, MODE == MODE_FIN ? row_bytes : 0u);
    const auto ro_r = rsrc(a.residual_out + tok_off, a.residual_out ? row_bytes : 0u);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float sh[8];
      Act<ACT>::unpack(shv[p], sh);
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = __builtin_fmaf(a.rsf, acc[p][e], sh[e]);
      const u32x4 s_pk = Act<ACT>::pack(sv);
      if constexpr (MODE == MODE_FIN) {
        __builtin_amdgcn_raw_buffer_store_b128(s_pk, fin_r, voff[p], 0, 0);
      } else {
        float s_r[8], res[8];
        Act<ACT>::unpack(s_pk, s_r);
        Act<ACT>::unpack(resv[p], res);
#pragma unroll
        for (int e = 0; e < 8; ++e) r[p][e] = s_r[e] + res[e];
        r_pk[p] = Act<ACT>::pack(r[p]);
        Act<ACT>::unpack(r_pk[p], r[p]);              // keep the rounded residual_out
        __builtin_amdgcn_raw_buffer_store_b128(r_pk[p], ro_r, voff[p], 0, NT);
        // lanes outside the row hold zeros here (all their loads read zeros)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(r[p][e], r[p][e], ss);
      }
    }
  }
  if constexpr (MODE == MODE_FIN) return;

  // ---- RMSNorm: sum of squares over the row (DPP within wavefronts, one LDS pass across,
  // then, for a split row, the slice partials of the token in slice order) ----
  __shared__ float wave_part[16];
  __shared__ float row_total;
  const int wave = tid >> 6;
  const int n_waves0 = L >> 6;                  // wavefronts of group 0
  if (g == 0) {
    const float ws = wave_sum(ss);
    if ((tid & 63) == 0) wave_part[wave] = ws;
  }
  lds_barrier();
  if (tid < 64) {                               // wavefront 0 of the workgroup
    // lane i reads wavefront i's partial (all reads in flight together); the partials are then
    // added in wavefront order through readlane, without waiting on LDS between the adds
    const float part = tid < n_waves0 ? wave_part[tid] : 0.f;
    float tot = 0.f;
    for (int i = 0; i < n_waves0; ++i)
      tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, part), i));
    if (a.slices > 1) {
      uint64_t* const slot = (uint64_t*)(a.ws + kWsHeader + (size_t)t * kWsPerToken);
      const int S = a.slices;
      const uint32_t epoch = epoch_prev + 1u;
      const int m = slice + tid * S;              // this slice's slots
      if (m < kMaxSlices) {
        const uint64_t v = ((uint64_t)epoch << 32) |
                           (m == slice ? (uint64_t)__builtin_bit_cast(uint32_t, tot) : 0ull);
        __hip_atomic_store(slot + m, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // lane j < S waits for slice j's word of this epoch; a partial that never arrives counts
      // as NaN
      uint32_t bits = 0;
      if (tid < S) {
        uint32_t spins = 0;
        while (true) {
          if (spins >= a.spin_limit) {
            __hip_atomic_fetch_or((uint32_t*)a.ws, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bits = kQuietNaN;
            break;
          }
          const uint64_t x = __hip_atomic_load(slot + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(x >> 32) == epoch) {
            bits = (uint32_t)x;
            break;
          }
          ++spins;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      tot = 0.f;
      for (int j = 0; j < S; ++j)                 // slice order: deterministic
        tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)bits, j));
    }
    if (tid == 0) row_total = tot;
  }
  lds_barrier();
  // NVFP4 with two or more route groups in at most four wavefronts (a.split_quant): group 1,
  // idle after the row sum, encodes elements 4..7 of every lane's slots from group 0's rounded
  // norm values (handed over in LDS) while group 0 encodes elements 0..3.
  constexpr bool kSplitQ = MODE == MODE_NVFP4 && G > 1;
  [[maybe_unused]] const bool split_q = kSplitQ && a.split_quant;
  [[maybe_unused]] const uint32_t qrow = MODE == MODE_FP8 ? (uint32_t)a.H : (uint32_t)a.H / 2u;
  [[maybe_unused]] const auto q_r =
      rsrc(a.quant_out + (int64_t)t * qrow, (MODE == MODE_FP8 || MODE == MODE_NVFP4) ? qrow : 0u);
  [[maybe_unused]] u32x4* const n_lds = (u32x4*)lds_dyn;
  if constexpr (kSplitQ) {
    if (split_q && g == 1) {
      lds_barrier();                            // group 0's rounded norm values are in LDS
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float nr[8];
        Act<ACT>::unpack(n_lds[p * L + lane], nr);
        quantize_store<MODE, NT, kSplitQ ? 2 : 0>(nr, qs, q_r, voff[p], live[p],
                                                  slot0 + lane + p * L, t,
                                                  QuantDst{a.sf_out, a.H, a.sf_swizzled});
      }
      return;
    }
  }
  if (g != 0) return;
  const float rinv = __builtin_amdgcn_rsqf(__builtin_fmaf(row_total, a.inv_h, a.eps));

  const auto no_r = rsrc(a.out + tok_off, a.out ? row_bytes : 0u);
  u32x4 n_pk[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float gm[8], n[8];
    Act<ACT>::unpack(gamv[p], gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = (r[p][e] * rinv) * gm[e];
    n_pk[p] = Act<ACT>::pack(n);
    __builtin_amdgcn_raw_buffer_store_b128(n_pk[p], no_r, voff[p], 0, NT);
    if constexpr (kSplitQ) {
      if (split_q) n_lds[p * L + lane] = n_pk[p];
    }
  }
  if constexpr (MODE == MODE_NVFP4 || MODE == MODE_FP8) {
    const QuantDst qd{a.sf_out, a.H, a.sf_swizzled};
    if (split_q) {
      lds_barrier();
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float nr[8];
        Act<ACT>::unpack(n_pk[p], nr);          // quantize the rounded norm_out values
        quantize_store<MODE, NT, kSplitQ ? 1 : 0>(nr, qs, q_r, voff[p], live[p],
                                                  slot0 + lane + p * L, t, qd);
      }
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float nr[8];
        Act<ACT>::unpack(n_pk[p], nr);
        quantize_store<MODE, NT, 0>(nr, qs, q_r, voff[p], live[p], slot0 + lane + p * L, t, qd);
      }
    }
  }
}

// Standalone quantizer: NVFP4 / FP8 of a given [T, H] activation tensor with the same device
// code as the fused epilogue. One wavefront per token and 512-element slice.
struct QuantParams {
  const uint8_t* x;
  const float* qscale;
  uint8_t* quant_out;
  uint8_t* sf_out;
  int T, H, nv, slices, sf_swizzled;
  int pad_blocks;   // workgroups after the T * slices quantizing ones that only zero scale padding
};

template <int ACT, int MODE>
__global__ __launch_bounds__(64) void quantize_kernel(const QuantParams a) {
  // the fields of the prologue in one batch of scalar loads, as in finalize_kernel
  asm volatile("" ::"s"(a.T), "s"(a.slices), "s"(a.H), "s"(a.nv), "s"(a.x));
  if constexpr (MODE == MODE_NVFP4) {
    // the swizzled layout's padding rows are zeroed by workgroups of their own, in parallel
    // with the quantizing ones (one workgroup per token and slice is too few at decode sizes)
    const int64_t n_main = (int64_t)a.T * a.slices;
    if (blockIdx.x >= n_main) {
      zero_sf_padding(QuantDst{a.sf_out, a.H, 1}, a.T, (blockIdx.x - n_main) * 64 + threadIdx.x,
                      (int64_t)a.pad_blocks * 64);
      return;
    }
  }
  const int t = blockIdx.x / a.slices;
  const int slice = blockIdx.x - t * a.slices;
  const int lane = threadIdx.x;
  const int s = slice * 64 + lane;
  const bool live = s < a.nv;
  const uint32_t voff = live ? (uint32_t)s * 16u : kOutOfRange;
  const uint32_t row_bytes = (uint32_t)a.H * 2u;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(a.x + (int64_t)t * row_bytes, row_bytes),
                                                        voff, 0, 0);
  // the row load goes out before the scale's: nothing waits for the scale ahead of the row
  __builtin_amdgcn_sched_barrier(0);
  const double qs = (double)*a.qscale;
  float xr[8];
  Act<ACT>::unpack(v, xr);
  const uint32_t qrow = MODE == MODE_FP8 ? (uint32_t)a.H : (uint32_t)a.H / 2u;
  const QuantDst d{a.sf_out, a.H, a.sf_swizzled};
  quantize_store<MODE>(xr, qs, rsrc(a.quant_out + (int64_t)t * qrow, qrow), voff, live, s, t, d);
}

// An empty kernel launched with a finalize entry point's grid, block and LDS: its duration is the
// launch-latency floor that the small-batch timings are reported against.
__global__ __launch_bounds__(1024) void launch_floor_kernel(int) {}

// Measurement aid: move n_rd 16-byte chunks in and n_wr chunks out in one launch, the way a
// perfect finalize would (every load of a round issued before any is used), with nothing else to
// do. Its time is the single-launch streaming ceiling for a given number of bytes, which the
// finalize timings are compared against. With `lanes` = grid x workgroup lanes, lane l reads, in
// rounds of LOADS loads in flight, every chunk c with c % lanes == l (round r: chunks
// l + (r * LOADS + i) * lanes), folds them with XOR, and stores the fold at every output chunk j
// with j % lanes == l; chunks past the end read zeros. NT = 2 makes every access nontemporal.
template <int LOADS, int NT>
__global__ __launch_bounds__(1024) void stream_probe_kernel(const uint8_t* src, uint32_t n_rd,
                                                            uint8_t* dst, uint32_t n_wr) {
  const uint32_t lanes = gridDim.x * blockDim.x;
  const uint32_t lane = blockIdx.x * blockDim.x + threadIdx.x;
  const auto rd = rsrc(src, n_rd * 16u);
  const auto wr = rsrc(dst, n_wr * 16u);
  u32x4 fold = {0u, 0u, 0u, 0u};
  for (uint32_t base = lane; base < n_rd; base += lanes * (uint32_t)LOADS) {
    u32x4 v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rd, (base + (uint32_t)i * lanes) * 16u, 0, NT);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) fold ^= v[i];
  }
  // every lane consumes its loads here, so none is moved into the store loop (which lanes past
  // the last output chunk skip)
  asm volatile("" ::"v"(fold));
  for (uint32_t j = lane; j < n_wr; j += lanes)
    __builtin_amdgcn_raw_buffer_store_b128(fold, wr, j * 16u, 0, NT);
}

// Zeroes n16 16-byte chunks at p (grid-stride): clears the static scratch of the allocation-free
// entry point on its first use on a device.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint8_t* p, uint32_t n16) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n16; i += stride)
    *(u32x4*)(p + (size_t)i * 16) = u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------------------------------------
// Host side: launch configuration and dispatch.
// ------------------------------------------------------------------------------------------------
struct Config {
  int G, P, JMAX, L, span, grid_x;
  size_t lds;
  bool nontemporal;
};

// Rows are read exactly once. Above 4 MiB of rows per call, nontemporal accesses to the streamed
// tensors (row, shared and residual loads; residual_out and norm_out stores) measured 5-18 %
// faster with the inputs in HBM (T = 64..256 at hidden 7168); below it they were no faster or
// slower, so small calls keep cacheable accesses (MOE_FIN_CACHE_AUTO). The caller may override
// the rule process-wide (moe_finalize_set_cache_policy); it is read when a call is enqueued.
constexpr int64_t kNontemporalRowBytes = (int64_t)4 << 20;
static std::atomic<int> g_cache_policy{MOE_FIN_CACHE_AUTO};
static bool use_nontemporal(int64_t T, int64_t H, int K) {
  switch (g_cache_policy.load(std::memory_order_relaxed)) {
    case MOE_FIN_CACHE_KEEP: return false;
    case MOE_FIN_CACHE_STREAM: return true;
  }
  return T * (int64_t)K * H * 2 >= kNontemporalRowBytes;
}

// Compute units of each device, queried once per device (hipDeviceAttributeMultiprocessorCount).
constexpr int kMaxDevices = 64;
static std::atomic<int> g_cus[kMaxDevices];
static int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FIN_ERR_HIP;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return MOE_FIN_ERR_HIP;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return MOE_FIN_OK;
}

// Polls of a split row's exchange word before a slice gives up (moe_finalize_set_wait_limit).
static std::atomic<uint32_t> g_spin_limit{kMaxSpins};

// Split rows of calls with cacheable accesses put the slices of a token on one XCD (workgroups
// are dealt to the 8 XCDs of gfx950 round-robin): the grid then has ceil(T / 8) * 8 * slices
// workgroups, those of tokens past T idle. Slices on consecutive XCDs start up to ~0.5 us
// apart (per-workgroup s_memrealtime timeline, T = 1 hidden 6144: 0.53 us median spread of the
// six slices' starts, 1.0 us median exchange), and the exchange waits for the last one.
// Same-box A/B, bit-identical outputs, top_k 8, median of replays:
//   inputs in the caches (the pages' protocol): T = 1 / 4 / 8 / 16 / 24 / 32 4.10 -> 3.74 /
//     4.19 -> 3.79 / 4.24 -> 3.95 / 4.12 -> 4.02 / 4.26 -> 4.06 / 4.28 -> 4.10 us; NVFP4 T = 1
//     4.79 -> 4.48; FP8 T = 16 4.60 -> 4.36;
//   inputs from HBM: T = 4 4.19 -> 3.94, but T = 8 / 16 / 24 / 32 / 64 +0.12 / +0.18 / +0.17 /
//     +0.21 / +0.36 us, T = 128 within 0.05.
// So the placement follows the cache policy's own assumption: calls with cacheable accesses
// (below 4 MiB of rows under AUTO; the decode batches a pipeline reads right after the expert
// GEMM wrote them) co-locate the slices; nontemporal calls (inputs assumed in HBM) do not.
constexpr int kXcds = 8;
static bool xcd_mapped(int mode, const Config& c) {
  return mode != 0 && c.grid_x > 1 && !c.nontemporal;
}
static int64_t main_blocks(int mode, const Config& c, int64_t T) {
  return xcd_mapped(mode, c) ? (T + kXcds - 1) / kXcds * kXcds * c.grid_x : (int64_t)c.grid_x * T;
}

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Route groups of the row modes (same-run A/B on MI355X over top_k 1..22, T = 1..256): the
// fewest groups that leave each group at most 4 routes (top_k 8: 2 groups of 4 routes beat 4
// groups of 2 by 0.15 us at decode and 0.44 us at T = 32; top_k 16 and 22: 4 groups of one
// wavefront beat 2 by 0.3-0.7 us), at least two wavefronts per workgroup when the routes allow
// it, and halved while the groups span more than 256 lanes unless a group would then carry more
// routes than max_routes; whole rows from 1024 tokens take one group up to top_k 48. Forced
// group counts, same box: split rows at top_k <= 8 with groups of 3-4 wavefronts (hidden
// 2560..7680 at decode, T = 48..64 at hidden 5120..7168) run 0.09-0.13 us faster warm and
// 0.26-0.55 us faster cold as one group; top_k 10 and 16 with
// groups of 2 wavefronts 0.02 / 0.20-0.36 us faster as 2 groups than 4; groups of 2 wavefronts
// at top_k 8 (the H6144 decode shapes, whole rows at hidden 1024) keep 2 groups, 0.10-0.15 us
// faster warm. Whole rows, cold: one group wins at top_k <= 16 (T = 256: 0.18-0.33 us, T = 512
// top_k 16: 1.4 us, T = 1024 top_k 16: 1.0-2.9 us), two at top_k 22 below 1024 tokens (T = 256 /
// 512: 0.22 / 1.85 us faster than four), one from 1024 tokens (top_k 10 / 22 / 33 at hidden
// 1024..2048: 3.1 / 4.0 / 5.3 us faster; top_k 64: 1.3 us faster at hidden 1024 but 2.1 us
// slower at hidden 2560, so top_k above 48 keeps the halving rule).
static void finish_config(int K, int64_t T, Config* c) {
  int G = 1;
  while (G < 4 && 2 * G * c->L <= 1024 && 2 * G <= K &&
         ((K + G - 1) / G > 4 || G * c->L < 128))
    G *= 2;
  if (c->grid_x == 1 && T >= 1024 && K <= 48) {
    G = 1;    // whole rows, several workgroups per CU: they hide the chunks of a single group
  } else {
    // routes a group may carry after halving: split rows 8, whole rows 16 (one chunk of loads)
    const int max_routes = c->grid_x > 1 ? 8 : 16;
    while (G > 1 && G * c->L > 256 && (K + G / 2 - 1) / (G / 2) <= max_routes) G /= 2;
  }
  c->G = G;
  const int J = (K + G - 1) / G;
  c->JMAX = next_pow2(J < 4 ? 4 : J);
  c->lds = (size_t)(G - 1) * c->P * c->L * 32;
}

// Slices per token for the split row modes, for a device of `cus` compute units. A CU keeps only
// so many vector memory requests in flight, so a whole row per workgroup leaves bandwidth unused
// when there are fewer tokens than CUs; splitting costs one cross-workgroup exchange (~1 us).
// Measured on MI355X, 256 CUs (forced slice counts, T = 1..256, hidden 1024..16384, top_k
// 6..22): up to top_k 8 the best slices hold at least 128 slots and give at most one workgroup
// per CU, min(slots / 128, CUs / T) (hidden 7168: 7 slices at T = 32, 4 at T = 64, 2 at
// T = 96..128, whole rows from T = 256); with more routes per token, smaller slices of 64 slots
// and ~7/8 of a workgroup per CU, min(slots / 64, (7/8) CUs / T), win, but
// no more than 16 of them (hidden 12288..16384 at T = 1..8: 16 slices beat 24-32 by 0.4-1.2 us,
// the exchange growing with the slices polled); with four routes or fewer (about five rows of
// data per token, e.g. a four-rank sum) whole rows win from T = 96 (0.14-0.16 us at T = 96 and
// 128, hidden 7168) for plain RMSNorm while a token's rows, shared and residual slices stay
// within 128 KiB for its CU (hidden 16384 top_k 4 split: 1.0-1.2 us faster at T = 96..128), while
// the quantized outputs keep the split: their epilogue is arithmetic-bound, and a whole row puts
// it on one CU (NVFP4 at T = 96..128, hidden 7168 and 16384: 1.1-2.2 us faster split; FP8
// 0.6-2.1 us, within 0.1 us at hidden 4096). 1 = whole rows (no workspace).
static int choose_slices(int64_t T, int nv, int K, bool quantized, int cus) {
  if (K <= 4 && T >= 96 && !quantized && (K + 2) * nv * 16 <= (128 << 10)) return 1;
  const int max_by_h = nv / (K > 8 ? 64 : 128);
  int S = (int)((K > 8 ? cus * 7 / 8 : cus) / (T > 0 ? T : 1));
  if (S > max_by_h) S = max_by_h;
  if (K > 8 && S > 16) S = 16;
  if (S > kMaxSlices) S = kMaxSlices;
  for (; S > 1; --S) {
    const int span = ((nv + S - 1) / S + 7) / 8 * 8;
    const int s_eff = (nv + span - 1) / span;
    if (s_eff == S) break;
  }
  return S < 1 ? 1 : S;
}

// Finalize-only: one workgroup per token and 64-slot slice, with route groups of at most 4
// routes each while the grid stays near 2048 wavefronts (G = 2 at K = 8 for small batches,
// G = 1 from T = 128, G = 4 at K >= 9 on small grids). Row modes: one workgroup per token and
// slice (slices = 1 covers the whole row with P slots per lane), route groups as finish_config
// chooses.
static bool make_config(int mode, int64_t T, int H, int K, int slices, Config* c) {
  const int nv = H / 8;
  c->nontemporal = false;
  if (mode == MODE_FIN) {
    c->P = 1;
    c->L = 64;
    c->span = 64;
    c->grid_x = (nv + 63) / 64;
    // the fewest route groups that leave each at most 4 routes (top_k 6: 2 groups, top_k 10:
    // 4 groups measured 0.2 us faster than 1 and 2; top_k 2 and 4 stay on one wavefront, which
    // beat two by 0.06-0.36 us), while the grid stays near 2048 wavefronts
    const int64_t waves = (T > 0 ? T : 1) * c->grid_x;
    int G = 1;
    while (G < 4 && (K + G - 1) / G > 4 && waves * 2 * G <= 2048) G *= 2;
    // Past the wavefront cap, one group of 17..24 routes loads its rows in two chunks; four
    // groups of at most 6 were as fast or faster at every measured size (cold, T = 64..1000,
    // hidden 4096..16384; top_k 17: T=100 H7168 7.76 -> 6.55 us, T=250 H4096 8.83 -> 7.73;
    // top_k 22: T=100 H16384 13.63 -> 12.28; top_k 24: T=1000 H16384 119.3 -> 117.7; worst
    // case top_k 17 T=1000 H16384 91.82 -> 91.96). top_k 25..32 (7-8 routes a group) measured
    // mixed (+0.1..0.2 us at T <= 250, -1.3..-3.5 us at T = 1000) and top_k 33 lost up to
    // 10 us at T = 1000, so both keep the cap.
    if ((K + G - 1) / G > 16 && K <= 24) G = 4;
    c->G = G;
    const int J = (K + G - 1) / G;
    c->JMAX = next_pow2(J < 4 ? 4 : J);
    c->lds = (size_t)(G - 1) * c->P * c->L * 32;
    return true;
  }
  if (slices > 1) {
    c->P = 1;
    c->span = ((nv + slices - 1) / slices + 7) / 8 * 8;
    c->L = (c->span + 63) / 64 * 64;
    c->grid_x = slices;
  } else {
    c->P = nv <= 1024 ? 1 : (nv <= 2048 ? 2 : 0);
    if (c->P == 0) return false;
    c->grid_x = 1;
    // From 1024 tokens, whole-row workgroups are rounded up to a multiple of four wavefronts
    // (one per SIMD; the extra lanes hold no slot). Measured on MI355X, cold, bit-identical
    // outputs: hidden 7168 top_k 8 T = 1024 / 2048 / 4096 -1.6 / -1.1 / -0.7 us, top_k 4
    // -1.4 us, hidden 3584 top_k 16 -1.8 us, hidden 5120 top_k 8 -0.9 / -1.2 us; neutral at
    // T = 256..768 and slower at T = 128..256 with top_k 4 (+0.15 us), where each CU holds one
    // workgroup and the idle wavefronts' predicated loads still occupy the address units. For
    // the same reason it is skipped when a route group carries more than 8 routes (more
    // registers, one workgroup per CU: hidden 7168 top_k 16 was 0.7 us slower).
    if (T >= 1024) {
      c->L = ((nv + c->P - 1) / c->P + 255) / 256 * 256;
      c->span = c->L * c->P;
      finish_config(K, T, c);
      if (c->JMAX <= 8) return true;
    }
    c->L = ((nv + c->P - 1) / c->P + 63) / 64 * 64;
    c->span = c->L * c->P;
  }
  finish_config(K, T, c);
  return true;
}

template <int ACT, int MODE, int G, int P, int JMAX>
static hipError_t launch_one(const Params& p, const Config& c, hipStream_t s) {
  dim3 grid((unsigned)(p.main_blocks + p.pad_blocks));
  dim3 block(c.G * c.L);
  if (c.nontemporal)
    hipLaunchKernelGGL((finalize_kernel<ACT, MODE, G, P, JMAX, 2>), grid, block, c.lds, s, p);
  else
    hipLaunchKernelGGL((finalize_kernel<ACT, MODE, G, P, JMAX, 0>), grid, block, c.lds, s, p);
  return hipGetLastError();
}

template <int ACT, int MODE, int G, int P>
static hipError_t dispatch_j(const Params& p, const Config& c, hipStream_t s) {
  switch (c.JMAX) {
    case 4: return launch_one<ACT, MODE, G, P, 4>(p, c, s);
    case 8: return launch_one<ACT, MODE, G, P, 8>(p, c, s);
    case 16: return launch_one<ACT, MODE, G, P, 16>(p, c, s);
    case 32:
      if constexpr (G <= 2) return launch_one<ACT, MODE, G, P, 32>(p, c, s);
      break;
    case 64:
      if constexpr (G == 1) return launch_one<ACT, MODE, G, P, 64>(p, c, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <int ACT, int MODE, int P>
static hipError_t dispatch_g(const Params& p, const Config& c, hipStream_t s) {
  switch (c.G) {
    case 1: return dispatch_j<ACT, MODE, 1, P>(p, c, s);
    case 2: return dispatch_j<ACT, MODE, 2, P>(p, c, s);
    case 4: return dispatch_j<ACT, MODE, 4, P>(p, c, s);
  }
  return hipErrorInvalidValue;
}

template <int ACT, int MODE>
static hipError_t dispatch_p(const Params& p, const Config& c, hipStream_t s) {
  if (c.P == 1) return dispatch_g<ACT, MODE, 1>(p, c, s);
  if constexpr (MODE != MODE_FIN) {
    if (c.P == 2) return dispatch_g<ACT, MODE, 2>(p, c, s);
  }
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t dispatch(int act, const Params& p, const Config& c, hipStream_t s) {
  return act == MOE_DTYPE_BF16 ? dispatch_p<ACT_BF16, MODE>(p, c, s)
                               : dispatch_p<ACT_FP16, MODE>(p, c, s);
}

// Whether the dispatch above has a kernel instantiation for this configuration (the same
// conditions as dispatch_p / dispatch_g / dispatch_j).
static bool kernel_available(int mode, const Config& c) {
  if (c.P != 1 && !(c.P == 2 && mode != MODE_FIN)) return false;
  if (c.G != 1 && c.G != 2 && c.G != 4) return false;
  switch (c.JMAX) {
    case 4: case 8: case 16: return true;
    case 32: return c.G <= 2;
    case 64: return c.G == 1;
  }
  return false;
}

// ---- argument checks ----------------------------------------------------------------------------
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;
};
static bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }
static Range rng(const void* p, size_t bytes) {
  return Range{(uintptr_t)p, (uintptr_t)p + bytes};
}

struct Common {
  const void* rows;
  int64_t n_rows;
  const int32_t* idx;
  const void* scales;
  int scales_dtype;
  const void* shared;
  float rsf;
  int64_t T, H;
  int K, act;
};

static int check_common(const Common& c, int h_multiple) {
  if (c.act != MOE_DTYPE_BF16 && c.act != MOE_DTYPE_FP16) return MOE_FIN_ERR_DTYPE;
  if (c.scales && c.scales_dtype != MOE_DTYPE_FP32 && c.scales_dtype != MOE_DTYPE_BF16)
    return MOE_FIN_ERR_DTYPE;
  if (c.K < 1 || c.K > 64) return MOE_FIN_ERR_BAD_TOPK;
  if (c.H <= 0 || c.H % h_multiple != 0) return MOE_FIN_ERR_HIDDEN;
  if (c.T < 0 || c.n_rows < 0) return MOE_FIN_ERR_BAD_SHAPE;
  if (c.T > INT32_MAX / 2 || c.H > (int64_t)1 << 20 || c.n_rows > INT32_MAX)
    return MOE_FIN_ERR_BAD_SHAPE;
  return MOE_FIN_OK;
}

static int check_pointers(const Common& c) {
  if (!c.idx || (c.n_rows > 0 && !c.rows)) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(c.rows, 16) || !aligned(c.idx, 4) || !aligned(c.shared, 16))
    return MOE_FIN_ERR_ALIGNMENT;
  if (c.scales && !aligned(c.scales, c.scales_dtype == MOE_DTYPE_FP32 ? 4 : 2))
    return MOE_FIN_ERR_ALIGNMENT;
  return MOE_FIN_OK;
}

// The reciprocal behind Params::slice_magic: m = ceil(2^32 / S) gives q / S = (q * m) >> 32 for
// every q with q * S < 2^32 (the error q * (m - 2^32 / S) / 2^32 stays below 1 / S); 0 where
// that does not hold for the workgroup indices below `grid` (the kernel divides then).
static uint32_t slice_reciprocal(int64_t S, int64_t grid) {
  if (S <= 1 || (uint64_t)grid * (uint64_t)S >= (1ull << 32)) return 0;
  return (uint32_t)(((1ull << 32) + (uint64_t)S - 1) / (uint64_t)S);
}

static Params base_params(const Common& c) {
  Params p;
  memset(&p, 0, sizeof(p));
  p.rows = (const uint8_t*)c.rows;
  p.n_rows = c.n_rows;
  p.idx = c.idx;
  p.scales = c.scales;
  p.scales_bf16 = c.scales_dtype == MOE_DTYPE_BF16;
  p.shared = (const uint8_t*)c.shared;
  p.rsf = c.rsf;
  p.T = (int)c.T;
  p.H = (int)c.H;
  p.K = c.K;
  p.nv = (int)(c.H / 8);
  p.inv_h = 1.0f / (float)c.H;
  return p;
}

static int to_code(hipError_t e) { return e == hipSuccess ? MOE_FIN_OK : MOE_FIN_ERR_HIP; }

// All inputs of the finalize, for the overlap checks against the outputs.
static int inputs_overlap(const Common& c, Range out) {
  const size_t e = 2;
  if (c.rows && overlap(out, rng(c.rows, (size_t)c.n_rows * c.H * e))) return 1;
  if (c.idx && overlap(out, rng(c.idx, (size_t)c.T * c.K * 4))) return 1;
  if (c.scales && overlap(out, rng(c.scales, (size_t)c.T * c.K *
                                                 (c.scales_dtype == MOE_DTYPE_FP32 ? 4 : 2))))
    return 1;
  if (c.shared && overlap(out, rng(c.shared, (size_t)c.T * c.H * e))) return 1;
  return 0;
}

static size_t workspace_bytes_for(int64_t T) { return kWsHeader + (size_t)T * kWsPerToken; }

// Scratch of moe_finalize_rmsnorm_noalloc_run: the split-row exchange words of up to
// kScratchTokens tokens in a file-scope device array, so that entry point allocates nothing and
// takes no workspace. Each device holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: the device address is obtained
// once per device with hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels.
constexpr int64_t kScratchTokens = 1024;
constexpr size_t kScratchBytes = kWsHeader + (size_t)kScratchTokens * kWsPerToken;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
static std::atomic<int> g_scratch_state[kMaxDevices];   // 0 new, 1 being set up, 2 ready

// The current device's scratch address. On the first call on a device it is looked up, and a
// kernel that zeroes the scratch is enqueued on `stream` ahead of the caller's work (the
// exchange protocol starts from a zero-filled state; a kernel rather than a memset node, so a
// graph captured around that first call replays correctly).
static int scratch_for_current_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FIN_ERR_HIP;
  if (g_scratch_state[dev].load(std::memory_order_acquire) != 2) {
    int expect = 0;
    if (!g_scratch_state[dev].compare_exchange_strong(expect, 1, std::memory_order_acq_rel)) {
      // another thread is setting this device up; wait for it (a few microseconds)
      while (g_scratch_state[dev].load(std::memory_order_acquire) == 1) {
      }
      if (g_scratch_state[dev].load(std::memory_order_acquire) != 2) return MOE_FIN_ERR_HIP;
    } else {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        g_scratch_state[dev].store(0, std::memory_order_release);
        return MOE_FIN_ERR_HIP;
      }
      hipLaunchKernelGGL(zero_fill_kernel, dim3(64), dim3(256), 0, stream, (uint8_t*)ptr,
                         (uint32_t)(kScratchBytes / 16));
      if (hipGetLastError() != hipSuccess) {
        g_scratch_state[dev].store(0, std::memory_order_release);
        return MOE_FIN_ERR_HIP;
      }
      g_scratch_ptr[dev].store((uint8_t*)ptr, std::memory_order_release);
      g_scratch_state[dev].store(2, std::memory_order_release);
    }
  }
  *out = g_scratch_ptr[dev].load(std::memory_order_acquire);
  return MOE_FIN_OK;
}

static int run_rows(int mode, const Common& c, const void* residual, const void* gamma,
                    float eps, void* residual_out, void* norm_out, const float* qscale,
                    void* quant_out, void* scale_out, int sf_layout, void* workspace,
                    void* stream, int route_stride = 0) {
  int slices = 1;
  if (workspace) {
    int cus = 0;
    const int rc = device_cus(&cus);
    if (rc) return rc;
    slices = choose_slices(c.T, (int)(c.H / 8), c.K, mode != MODE_RMS, cus);
  }
  Config cfg;
  if (!make_config(mode, c.T, (int)c.H, c.K, slices, &cfg)) return MOE_FIN_ERR_HIDDEN;
  cfg.nontemporal = use_nontemporal(c.T, c.H, c.K);
  // swizzled NVFP4 with padding rows: workgroups after the token ones that zero the padding
  // scale bytes, about two 4-byte words per thread
  const int pad_blocks =
      mode == MODE_NVFP4 && sf_layout == MOE_SF_SWIZZLED_128x4 && c.T % 128 != 0
          ? (int)((((c.H / 16 + 3) / 4) * 128 + 2 * cfg.G * cfg.L - 1) / (2 * cfg.G * cfg.L))
          : 0;
  const int64_t n_main = main_blocks(mode, cfg, c.T);
  if (n_main + pad_blocks > INT32_MAX) return MOE_FIN_ERR_BAD_SHAPE;
  Params p = base_params(c);
  p.residual = (const uint8_t*)residual;
  p.gamma = (const uint8_t*)gamma;
  p.eps = eps;
  p.residual_out = (uint8_t*)residual_out;
  p.out = (uint8_t*)norm_out;
  p.quant_out = (uint8_t*)quant_out;
  p.sf_out = (uint8_t*)scale_out;
  p.qscale = qscale;
  p.sf_swizzled = sf_layout == MOE_SF_SWIZZLED_128x4;
  p.lanes = cfg.L;
  p.slot_span = cfg.span;
  p.slices = cfg.grid_x;
  p.main_blocks = (int)n_main;
  p.slice_magic = slice_reciprocal(p.slices, n_main);
  p.xcd_map = xcd_mapped(mode, cfg) ? 1 : 0;
  p.ws = (uint8_t*)workspace;
  p.route_stride = route_stride;
  p.pad_blocks = pad_blocks;
  p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  // Half of the NVFP4 codes go to route group 1 when the workgroup has at most four wavefronts,
  // so each wavefront of the epilogue has a SIMD of its own. Same-box A/B, bit-identical
  // outputs, hidden 6144 top_k 8: NVFP4 T = 1 / 16 4.75 -> 4.62 / 4.97 -> 4.81 us (two groups of
  // two wavefronts); at T = 64 (two groups of three) it cost 0.08-0.10 us, and FP8, whose codes
  // cost less, lost 0.05 us at T = 1.
  p.split_quant = mode == MODE_NVFP4 && cfg.G >= 2 && cfg.G * cfg.L <= 256;
  hipStream_t s = (hipStream_t)stream;
  switch (mode) {
    case MODE_RMS: return to_code(dispatch<MODE_RMS>(c.act, p, cfg, s));
    case MODE_NVFP4: return to_code(dispatch<MODE_NVFP4>(c.act, p, cfg, s));
    case MODE_FP8: return to_code(dispatch<MODE_FP8>(c.act, p, cfg, s));
  }
  return MOE_FIN_ERR_QUANT_TYPE;
}

// Validation shared by the residual + RMSNorm entry points.
static int check_rows(const Common& c, const void* residual, const void* gamma,
                      const void* residual_out, const void* norm_out, bool norm_required) {
  if (!residual || !gamma || (norm_required && !norm_out)) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) ||
      !aligned(norm_out, 16))
    return MOE_FIN_ERR_ALIGNMENT;
  const size_t tb = (size_t)c.T * c.H * 2;
  if (norm_out) {
    Range o = rng(norm_out, tb);
    if (inputs_overlap(c, o) || overlap(o, rng(residual, tb)) ||
        overlap(o, rng(gamma, (size_t)c.H * 2)))
      return MOE_FIN_ERR_ALIAS;
    if (residual_out && overlap(o, rng(residual_out, tb))) return MOE_FIN_ERR_ALIAS;
  }
  if (residual_out) {
    Range o = rng(residual_out, tb);
    if (inputs_overlap(c, o) || overlap(o, rng(gamma, (size_t)c.H * 2)))
      return MOE_FIN_ERR_ALIAS;
    if (residual_out != residual && overlap(o, rng(residual, tb))) return MOE_FIN_ERR_ALIAS;
  }
  return MOE_FIN_OK;
}

// Workspace of the split row modes: NULL (whole rows) or at least workspace_bytes_for(T) bytes,
// 256-byte aligned, overlapping no other buffer.
static int check_workspace(const Common& c, const void* ws, size_t ws_bytes,
                           std::initializer_list<Range> others) {
  if (!ws) return MOE_FIN_OK;
  if (!aligned(ws, 256)) return MOE_FIN_ERR_ALIGNMENT;
  if (ws_bytes < workspace_bytes_for(c.T)) return MOE_FIN_ERR_WORKSPACE;
  Range w = rng(ws, ws_bytes);
  if (inputs_overlap(c, w)) return MOE_FIN_ERR_ALIAS;
  for (const Range& o : others)
    if (o.hi > o.lo && overlap(w, o)) return MOE_FIN_ERR_ALIAS;
  return MOE_FIN_OK;
}

// The residual + RMSNorm entry points after their own shape checks: rows (with a route map,
// route_stride == 0) or strided rows (route_stride = T: route k of token t is row k*T + t, no map).
static int rmsnorm_call(const Common& c, const void* residual, const void* gamma, float eps,
                        void* residual_out, void* norm_out, void* workspace,
                        size_t workspace_bytes, void* stream, int route_stride) {
  if (c.H > 16384) return MOE_FIN_ERR_HIDDEN;
  if (c.T == 0) return MOE_FIN_OK;
  int rc;
  if (route_stride == 0) {
    if ((rc = check_pointers(c))) return rc;
  } else {
    if (!c.rows) return MOE_FIN_ERR_NULL_POINTER;
    if (!aligned(c.rows, 16)) return MOE_FIN_ERR_ALIGNMENT;
  }
  if ((rc = check_rows(c, residual, gamma, residual_out, norm_out, true))) return rc;
  const size_t tb = (size_t)c.T * c.H * 2;
  if ((rc = check_workspace(c, workspace, workspace_bytes,
                            {rng(residual, tb), rng(gamma, (size_t)c.H * 2),
                             residual_out ? rng(residual_out, tb) : Range{0, 0},
                             rng(norm_out, tb)})))
    return rc;
  return run_rows(MODE_RMS, c, residual, gamma, eps, residual_out, norm_out, nullptr, nullptr,
                  nullptr, 0, workspace, stream, route_stride);
}

// The quantized entry points, likewise.
static int quant_call(const Common& c, const void* residual, const void* gamma, float eps,
                      int quant_type, const float* quant_scale, void* quant_out, void* scale_out,
                      int sf_layout, void* residual_out, void* norm_out, void* workspace,
                      size_t workspace_bytes, void* stream, int route_stride) {
  if (quant_type != MOE_QUANT_NVFP4 && quant_type != MOE_QUANT_FP8_E4M3)
    return MOE_FIN_ERR_QUANT_TYPE;
  const bool nvfp4 = quant_type == MOE_QUANT_NVFP4;
  if (nvfp4 && sf_layout != MOE_SF_LINEAR && sf_layout != MOE_SF_SWIZZLED_128x4)
    return MOE_FIN_ERR_SF_LAYOUT;
  int rc = check_common(c, nvfp4 ? 16 : 8);
  if (rc) return rc;
  if (c.H > 16384) return MOE_FIN_ERR_HIDDEN;
  if (c.T == 0) return MOE_FIN_OK;
  if (route_stride == 0) {
    if ((rc = check_pointers(c))) return rc;
  } else {
    if (!c.rows) return MOE_FIN_ERR_NULL_POINTER;
    if (!aligned(c.rows, 16)) return MOE_FIN_ERR_ALIGNMENT;
  }
  if ((rc = check_rows(c, residual, gamma, residual_out, norm_out, false))) return rc;
  if (!quant_scale || !quant_out || (nvfp4 && !scale_out)) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(quant_scale, 4) || !aligned(quant_out, 16) || (nvfp4 && !aligned(scale_out, 4)))
    return MOE_FIN_ERR_ALIGNMENT;
  const size_t qbytes = (size_t)c.T * c.H / (nvfp4 ? 2 : 1);
  const size_t sbytes = nvfp4 ? moe_finalize_sf_size(c.T, c.H, sf_layout) : 0;
  const size_t tb = (size_t)c.T * c.H * 2;
  Range q = rng(quant_out, qbytes);
  if (inputs_overlap(c, q) || overlap(q, rng(residual, tb)) ||
      overlap(q, rng(gamma, (size_t)c.H * 2)) ||
      (residual_out && overlap(q, rng(residual_out, tb))) ||
      (norm_out && overlap(q, rng(norm_out, tb))) || overlap(q, rng(quant_scale, 4)))
    return MOE_FIN_ERR_ALIAS;
  if (nvfp4) {
    Range sr = rng(scale_out, sbytes);
    if (inputs_overlap(c, sr) || overlap(sr, q) || overlap(sr, rng(residual, tb)) ||
        overlap(sr, rng(gamma, (size_t)c.H * 2)) ||
        (residual_out && overlap(sr, rng(residual_out, tb))) ||
        (norm_out && overlap(sr, rng(norm_out, tb))) || overlap(sr, rng(quant_scale, 4)))
      return MOE_FIN_ERR_ALIAS;
  }
  if ((rc = check_workspace(c, workspace, workspace_bytes,
                            {rng(residual, tb), rng(gamma, (size_t)c.H * 2),
                             residual_out ? rng(residual_out, tb) : Range{0, 0},
                             norm_out ? rng(norm_out, tb) : Range{0, 0}, q,
                             nvfp4 ? rng(scale_out, sbytes) : Range{0, 0},
                             rng(quant_scale, 4)})))
    return rc;
  return run_rows(nvfp4 ? MODE_NVFP4 : MODE_FP8, c, residual, gamma, eps, residual_out, norm_out,
                  quant_scale, quant_out, scale_out, sf_layout, workspace, stream, route_stride);
}

}  // namespace mfin

using namespace mfin;

extern "C" {

int moe_finalize_version(void) { return 300; }

int64_t moe_finalize_set_wait_limit(int64_t polls) {
  const uint32_t v = polls < 0 ? kMaxSpins
                               : (polls > (int64_t)UINT32_MAX ? UINT32_MAX : (uint32_t)polls);
  return (int64_t)g_spin_limit.exchange(v);
}

int moe_finalize_set_cache_policy(int policy) {
  if (policy != MOE_FIN_CACHE_AUTO && policy != MOE_FIN_CACHE_KEEP &&
      policy != MOE_FIN_CACHE_STREAM)
    return MOE_FIN_ERR_POLICY;
  return g_cache_policy.exchange(policy);
}

const char* moe_finalize_error_string(int code) {
  switch (code) {
    case MOE_FIN_OK: return "success";
    case MOE_FIN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MOE_FIN_ERR_BAD_SHAPE: return "negative or oversized num_tokens / num_permuted_rows";
    case MOE_FIN_ERR_BAD_TOPK: return "top_k outside [1, 64]";
    case MOE_FIN_ERR_HIDDEN:
      return "hidden must be positive and a multiple of 8 (16 for NVFP4), at most 16384 for the "
             "RMSNorm entry points";
    case MOE_FIN_ERR_ALIGNMENT: return "a pointer is not aligned as required";
    case MOE_FIN_ERR_DTYPE: return "unknown act_dtype or scales_dtype";
    case MOE_FIN_ERR_QUANT_TYPE: return "unknown quant_type";
    case MOE_FIN_ERR_SF_LAYOUT: return "scale layout must be LINEAR or SWIZZLED_128x4";
    case MOE_FIN_ERR_ALIAS: return "an output overlaps an input or another output";
    case MOE_FIN_ERR_HIP: return "the HIP runtime refused the kernel launch";
    case MOE_FIN_ERR_WORKSPACE:
      return "workspace smaller than moe_finalize_workspace_size(num_tokens, hidden, top_k)";
    case MOE_FIN_ERR_POLICY: return "unknown cache policy";
    case MOE_FIN_ERR_SCRATCH:
      return "num_tokens above the 1024 that moe_finalize_rmsnorm_noalloc_run's static scratch "
             "holds";
  }
  return "unknown error code";
}

size_t moe_finalize_sf_size(int64_t num_tokens, int64_t hidden, int sf_layout) {
  if (num_tokens < 0 || hidden < 0) return 0;
  const int64_t nb = hidden / 16;
  if (sf_layout == MOE_SF_SWIZZLED_128x4)
    return (size_t)((num_tokens + 127) / 128 * 128) * (size_t)((nb + 3) / 4 * 4);
  if (sf_layout == MOE_SF_LINEAR) return (size_t)(num_tokens * nb);
  return 0;
}

size_t moe_finalize_workspace_size(int64_t num_tokens, int64_t hidden, int top_k) {
  (void)hidden;
  (void)top_k;
  if (num_tokens < 0) return 0;
  return workspace_bytes_for(num_tokens);
}

// The launch configuration of entry point `entry` (0 = finalize, 1 = RMSNorm, 2 = quantized) for
// one shape, with the entry point's own shape checks.
static int entry_config(int entry, int64_t num_tokens, int64_t hidden, int top_k,
                        bool with_workspace, int num_cus, Config* c) {
  if (entry < 0 || entry > 2) return MOE_FIN_ERR_QUANT_TYPE;
  if (top_k < 1 || top_k > 64) return MOE_FIN_ERR_BAD_TOPK;
  if (hidden <= 0 || hidden % 8 != 0 || (entry > 0 && hidden > 16384)) return MOE_FIN_ERR_HIDDEN;
  if (num_tokens < 0 || num_tokens > INT32_MAX / 2) return MOE_FIN_ERR_BAD_SHAPE;
  const int64_t T = num_tokens > 0 ? num_tokens : 1;
  int slices = 1;
  if (entry > 0 && with_workspace) {
    int cus = num_cus;
    if (cus <= 0) {
      const int rc = device_cus(&cus);
      if (rc) return rc;
    }
    slices = choose_slices(T, (int)(hidden / 8), top_k, entry == 2, cus);
  }
  if (!make_config(entry == 0 ? MODE_FIN : MODE_RMS, T, (int)hidden, top_k, slices, c))
    return MOE_FIN_ERR_HIDDEN;
  c->nontemporal = use_nontemporal(T, hidden, top_k);
  if (main_blocks(entry == 0 ? MODE_FIN : MODE_RMS, *c, T) > INT32_MAX) return MOE_FIN_ERR_BAD_SHAPE;
  return MOE_FIN_OK;
}

int moe_finalize_launch_floor_run(int entry, int64_t num_tokens, int64_t hidden, int top_k,
                                  void* stream) {
  Config c;
  // (T = 0 only validates the shape: no slice rule, so no device query)
  const int rc = entry_config(entry, num_tokens, hidden, top_k, num_tokens > 0, 0, &c);
  if (rc || num_tokens == 0) return rc;
  hipLaunchKernelGGL(launch_floor_kernel,
                     dim3((unsigned)main_blocks(entry == 0 ? MODE_FIN : MODE_RMS, c, num_tokens)),
                     dim3(c.G * c.L),
                     c.lds, (hipStream_t)stream, 0);
  return to_code(hipGetLastError());
}

int moe_finalize_launch_config(int entry, int64_t num_tokens, int64_t hidden, int top_k,
                               int with_workspace, int num_cus, int64_t* out, int n_out) {
  if (!out) return MOE_FIN_ERR_NULL_POINTER;
  if (n_out < MOE_FIN_LAUNCH_CONFIG_FIELDS) return MOE_FIN_ERR_BAD_SHAPE;
  Config c;
  const int rc =
      entry_config(entry, num_tokens, hidden, top_k, with_workspace != 0, num_cus, &c);
  if (rc) return rc;
  out[0] = num_tokens > 0 ? main_blocks(entry == 0 ? MODE_FIN : MODE_RMS, c, num_tokens) : 0;
  out[1] = (int64_t)c.G * c.L;
  out[2] = entry > 0 ? c.grid_x : 1;
  out[3] = c.G;
  out[4] = c.P;
  out[5] = c.span;
  out[6] = (int64_t)c.lds;
  out[7] = c.nontemporal ? 1 : 0;
  out[8] = kernel_available(entry == 0 ? MODE_FIN : MODE_RMS, c) ? 1 : 0;
  return MOE_FIN_OK;
}

// Shape checks and launch of the stream probe (both measurement entry points).
static int stream_probe(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                        int loads, int lanes, int64_t grid, int nontemporal, void* stream) {
  const size_t kMax = (size_t)1 << 31;
  if (read_bytes % 16 != 0 || write_bytes % 16 != 0 || read_bytes > kMax || write_bytes > kMax)
    return MOE_FIN_ERR_BAD_SHAPE;
  if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return MOE_FIN_ERR_BAD_SHAPE;
  if (lanes != 64 && lanes != 128 && lanes != 256 && lanes != 512 && lanes != 1024)
    return MOE_FIN_ERR_BAD_SHAPE;
  if (grid < 1 || grid > 65536) return MOE_FIN_ERR_BAD_SHAPE;
  // every chunk offset a lane forms, base + i * lanes < 2^27 + 2^27 chunks, stays below 2^32 bytes
  if (grid * lanes * loads > ((int64_t)1 << 27)) return MOE_FIN_ERR_BAD_SHAPE;
  if ((read_bytes && !src) || (write_bytes && !dst)) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_FIN_ERR_ALIGNMENT;
  if (read_bytes && write_bytes && overlap(rng(src, read_bytes), rng(dst, write_bytes)))
    return MOE_FIN_ERR_ALIAS;
  const uint32_t n_rd = (uint32_t)(read_bytes / 16), n_wr = (uint32_t)(write_bytes / 16);
  if (n_rd == 0 && n_wr == 0) return MOE_FIN_OK;
  const dim3 g((unsigned)grid), b((unsigned)lanes);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* sp = (const uint8_t*)src;
  uint8_t* dp = (uint8_t*)dst;
#define MFIN_PROBE(L)                                                                          \
  case L:                                                                                      \
    if (nontemporal)                                                                           \
      hipLaunchKernelGGL((stream_probe_kernel<L, 2>), g, b, 0, s, sp, n_rd, dp, n_wr);         \
    else                                                                                       \
      hipLaunchKernelGGL((stream_probe_kernel<L, 0>), g, b, 0, s, sp, n_rd, dp, n_wr);         \
    break;
  switch (loads) {
    MFIN_PROBE(1)
    MFIN_PROBE(2)
    MFIN_PROBE(4)
    MFIN_PROBE(8)
    MFIN_PROBE(16)
  }
#undef MFIN_PROBE
  return to_code(hipGetLastError());
}

// The fastest shape of a cold launch-shape sweep on MI355X at 9.2 and 18.4 MB (loads per round
// 1..16, 256..1024-lane workgroups, 256..3590 workgroups, nontemporal or not): one load per round,
// four 512-lane workgroups per CU, nontemporal. 18.4 MB: 4.28 us against 4.45 for the next shape
// and 4.61 for one round of four loads in 256-lane workgroups; 9.2 MB: 2.88 us, within 0.02 us
// of the best.
int moe_finalize_stream_floor_run(const void* src, size_t read_bytes, void* dst,
                                  size_t write_bytes, void* stream) {
  return stream_probe(src, read_bytes, dst, write_bytes, 1, 512, 1024, 1, stream);
}

int moe_finalize_stream_probe_run(const void* src, size_t read_bytes, void* dst,
                                  size_t write_bytes, int loads_per_round, int workgroup_lanes,
                                  int64_t workgroups, int nontemporal, void* stream) {
  return stream_probe(src, read_bytes, dst, write_bytes, loads_per_round, workgroup_lanes,
                      workgroups, nontemporal, stream);
}

int moe_finalize_run(const void* permuted_rows, int64_t num_permuted_rows,
                     const int32_t* expanded_idx_to_permuted_idx, const void* expert_scales,
                     int scales_dtype, const void* shared_expert_output,
                     float routed_scaling_factor, void* out, int64_t num_tokens, int64_t hidden,
                     int top_k, int act_dtype, void* stream) {
  Common c{permuted_rows, num_permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
           scales_dtype, shared_expert_output, routed_scaling_factor, num_tokens, hidden,
           top_k, act_dtype};
  int rc = check_common(c, 8);
  if (rc) return rc;
  if (num_tokens == 0) return MOE_FIN_OK;
  if ((rc = check_pointers(c))) return rc;
  if (!out) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(out, 16)) return MOE_FIN_ERR_ALIGNMENT;
  if (inputs_overlap(c, rng(out, (size_t)num_tokens * hidden * 2))) return MOE_FIN_ERR_ALIAS;
  Config cfg;
  make_config(MODE_FIN, num_tokens, (int)hidden, top_k, 1, &cfg);
  cfg.nontemporal = use_nontemporal(num_tokens, hidden, top_k);
  if ((int64_t)cfg.grid_x * num_tokens > INT32_MAX) return MOE_FIN_ERR_BAD_SHAPE;
  Params p = base_params(c);
  p.main_blocks = (int)(cfg.grid_x * num_tokens);
  p.out = (uint8_t*)out;
  p.lanes = cfg.L;
  p.slot_span = cfg.span;
  p.slices = cfg.grid_x;
  p.slice_magic = slice_reciprocal(p.slices, p.main_blocks);
  return to_code(dispatch<MODE_FIN>(act_dtype, p, cfg, (hipStream_t)stream));
}

int moe_finalize_rmsnorm_run(const void* permuted_rows, int64_t num_permuted_rows,
                             const int32_t* expanded_idx_to_permuted_idx,
                             const void* expert_scales, int scales_dtype,
                             const void* shared_expert_output, float routed_scaling_factor,
                             const void* residual, const void* gamma, float eps,
                             void* residual_out, void* norm_out, void* workspace,
                             size_t workspace_bytes, int64_t num_tokens, int64_t hidden,
                             int top_k, int act_dtype, void* stream) {
  Common c{permuted_rows, num_permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
           scales_dtype, shared_expert_output, routed_scaling_factor, num_tokens, hidden,
           top_k, act_dtype};
  const int rc = check_common(c, 8);
  if (rc) return rc;
  return rmsnorm_call(c, residual, gamma, eps, residual_out, norm_out, workspace,
                      workspace_bytes, stream, 0);
}

int moe_finalize_rmsnorm_noalloc_run(const void* permuted_rows, int64_t num_permuted_rows,
                                     const int32_t* expanded_idx_to_permuted_idx,
                                     const void* expert_scales, int scales_dtype,
                                     const void* shared_expert_output,
                                     float routed_scaling_factor, const void* residual,
                                     const void* gamma, float eps, void* residual_out,
                                     void* norm_out, int64_t num_tokens, int64_t hidden,
                                     int top_k, int act_dtype, void* stream) {
  Common c{permuted_rows, num_permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
           scales_dtype, shared_expert_output, routed_scaling_factor, num_tokens, hidden,
           top_k, act_dtype};
  int rc = check_common(c, 8);
  if (rc) return rc;
  if (num_tokens > kScratchTokens) return MOE_FIN_ERR_SCRATCH;
  if (hidden > 16384) return MOE_FIN_ERR_HIDDEN;
  if (num_tokens == 0) return MOE_FIN_OK;
  if ((rc = check_pointers(c))) return rc;
  if ((rc = check_rows(c, residual, gamma, residual_out, norm_out, true))) return rc;
  uint8_t* ws = nullptr;
  if ((rc = scratch_for_current_device((hipStream_t)stream, &ws))) return rc;
  return run_rows(MODE_RMS, c, residual, gamma, eps, residual_out, norm_out, nullptr, nullptr,
                  nullptr, 0, ws, stream, 0);
}

int moe_finalize_workspace_flag(const void* workspace, int clear, int* flag, void* stream) {
  if (!flag) return MOE_FIN_ERR_NULL_POINTER;
  const void* src = workspace;
  if (!src) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FIN_ERR_HIP;
    // the static scratch of moe_finalize_rmsnorm_noalloc_run; never used yet on this device: 0
    if (g_scratch_state[dev].load(std::memory_order_acquire) != 2) {
      *flag = 0;
      return MOE_FIN_OK;
    }
    src = g_scratch_ptr[dev].load(std::memory_order_acquire);
  } else if (!aligned(workspace, 256)) {
    return MOE_FIN_ERR_ALIGNMENT;
  }
  uint32_t v = 0;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&v, src, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_FIN_ERR_HIP;
  *flag = (int)v;
  if (clear && v) {
    // the flag's 16-byte unit of the header; the rest of the header is unused
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1), dim3(256), 0, s, (uint8_t*)src, 1u);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
      return MOE_FIN_ERR_HIP;
  }
  return MOE_FIN_OK;
}

int moe_residual_rmsnorm_run(const void* x, const void* residual, const void* gamma, float eps,
                             void* residual_out, void* norm_out, void* workspace,
                             size_t workspace_bytes, int64_t num_tokens, int64_t hidden,
                             int act_dtype, void* stream) {
  // The residual + RMSNorm of the finalize path on a given x: the finalize with one route per
  // token (row t of x, weight 1), RSF 1 and no shared term reproduces x exactly.
  Common c{x, num_tokens, nullptr, nullptr, MOE_DTYPE_FP32, nullptr, 1.0f, num_tokens, hidden,
           1, act_dtype};
  const int rc = check_common(c, 8);
  if (rc) return rc;
  return rmsnorm_call(c, residual, gamma, eps, residual_out, norm_out, workspace,
                      workspace_bytes, stream, (int)num_tokens);
}

int moe_rank_sum_rmsnorm_run(const void* rank_partials, int world_size, const void* residual,
                             const void* gamma, float eps, void* residual_out, void* norm_out,
                             void* workspace, size_t workspace_bytes, int64_t num_tokens,
                             int64_t hidden, int act_dtype, void* stream) {
  // The rank sum is the finalize with one route per rank (row r*T + t, weight 1), RSF 1 and no
  // shared term: the float32 sum of the W partials, rounded once.
  Common c{rank_partials, (int64_t)world_size * num_tokens, nullptr, nullptr, MOE_DTYPE_FP32,
           nullptr, 1.0f, num_tokens, hidden, world_size, act_dtype};
  const int rc = check_common(c, 8);
  if (rc) return rc;
  return rmsnorm_call(c, residual, gamma, eps, residual_out, norm_out, workspace,
                      workspace_bytes, stream, (int)num_tokens);
}

int moe_rank_sum_quant_run(const void* rank_partials, int world_size, const void* residual,
                           const void* gamma, float eps, int quant_type, const float* quant_scale,
                           void* quant_out, void* scale_out, int sf_layout, void* residual_out,
                           void* norm_out, void* workspace, size_t workspace_bytes,
                           int64_t num_tokens, int64_t hidden, int act_dtype, void* stream) {
  Common c{rank_partials, (int64_t)world_size * num_tokens, nullptr, nullptr, MOE_DTYPE_FP32,
           nullptr, 1.0f, num_tokens, hidden, world_size, act_dtype};
  return quant_call(c, residual, gamma, eps, quant_type, quant_scale, quant_out, scale_out,
                    sf_layout, residual_out, norm_out, workspace, workspace_bytes, stream,
                    (int)num_tokens);
}

int moe_quantize_run(const void* x, int64_t num_tokens, int64_t hidden, int act_dtype,
                     int quant_type, const float* quant_scale, void* quant_out, void* scale_out,
                     int sf_layout, void* stream) {
  if (act_dtype != MOE_DTYPE_BF16 && act_dtype != MOE_DTYPE_FP16) return MOE_FIN_ERR_DTYPE;
  if (quant_type != MOE_QUANT_NVFP4 && quant_type != MOE_QUANT_FP8_E4M3)
    return MOE_FIN_ERR_QUANT_TYPE;
  const bool nvfp4 = quant_type == MOE_QUANT_NVFP4;
  if (nvfp4 && sf_layout != MOE_SF_LINEAR && sf_layout != MOE_SF_SWIZZLED_128x4)
    return MOE_FIN_ERR_SF_LAYOUT;
  if (hidden <= 0 || hidden % (nvfp4 ? 16 : 8) != 0 || hidden > ((int64_t)1 << 20))
    return MOE_FIN_ERR_HIDDEN;
  if (num_tokens < 0 || num_tokens > INT32_MAX / 2) return MOE_FIN_ERR_BAD_SHAPE;
  if (num_tokens == 0) return MOE_FIN_OK;
  if (!x || !quant_scale || !quant_out || (nvfp4 && !scale_out)) return MOE_FIN_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(quant_scale, 4) || !aligned(quant_out, 16) ||
      (nvfp4 && !aligned(scale_out, 4)))
    return MOE_FIN_ERR_ALIGNMENT;
  const size_t xb = (size_t)num_tokens * hidden * 2;
  const Range q = rng(quant_out, (size_t)num_tokens * hidden / (nvfp4 ? 2 : 1));
  if (overlap(q, rng(x, xb)) || overlap(q, rng(quant_scale, 4))) return MOE_FIN_ERR_ALIAS;
  if (nvfp4) {
    const Range sr = rng(scale_out, moe_finalize_sf_size(num_tokens, hidden, sf_layout));
    if (overlap(sr, rng(x, xb)) || overlap(sr, q) || overlap(sr, rng(quant_scale, 4)))
      return MOE_FIN_ERR_ALIAS;
  }
  QuantParams p;
  p.x = (const uint8_t*)x;
  p.qscale = quant_scale;
  p.quant_out = (uint8_t*)quant_out;
  p.sf_out = (uint8_t*)scale_out;
  p.T = (int)num_tokens;
  p.H = (int)hidden;
  p.nv = (int)(hidden / 8);
  p.slices = (p.nv + 63) / 64;
  p.sf_swizzled = sf_layout == MOE_SF_SWIZZLED_128x4;
  // padding rows (swizzled NVFP4, T not a multiple of 128): about two words per thread
  p.pad_blocks = nvfp4 && p.sf_swizzled && (num_tokens % 128) != 0
                     ? (int)((((hidden / 16 + 3) / 4) * 128 + 127) / 128)
                     : 0;
  if ((int64_t)p.slices * num_tokens + p.pad_blocks > INT32_MAX) return MOE_FIN_ERR_BAD_SHAPE;
  const dim3 grid((unsigned)(p.slices * num_tokens + p.pad_blocks)), block(64);
  hipStream_t s = (hipStream_t)stream;
  if (act_dtype == MOE_DTYPE_BF16) {
    if (nvfp4) hipLaunchKernelGGL((quantize_kernel<ACT_BF16, MODE_NVFP4>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((quantize_kernel<ACT_BF16, MODE_FP8>), grid, block, 0, s, p);
  } else {
    if (nvfp4) hipLaunchKernelGGL((quantize_kernel<ACT_FP16, MODE_NVFP4>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((quantize_kernel<ACT_FP16, MODE_FP8>), grid, block, 0, s, p);
  }
  return to_code(hipGetLastError());
}

int moe_finalize_quant_run(const void* permuted_rows, int64_t num_permuted_rows,
                           const int32_t* expanded_idx_to_permuted_idx, const void* expert_scales,
                           int scales_dtype, const void* shared_expert_output,
                           float routed_scaling_factor, const void* residual, const void* gamma,
                           float eps, int quant_type, const float* quant_scale, void* quant_out,
                           void* scale_out, int sf_layout, void* residual_out, void* norm_out,
                           void* workspace, size_t workspace_bytes, int64_t num_tokens,
                           int64_t hidden, int top_k, int act_dtype, void* stream) {
  Common c{permuted_rows, num_permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
           scales_dtype, shared_expert_output, routed_scaling_factor, num_tokens, hidden,
           top_k, act_dtype};
  return quant_call(c, residual, gamma, eps, quant_type, quant_scale, quant_out, scale_out,
                    sf_layout, residual_out, norm_out, workspace, workspace_bytes, stream, 0);
}

}  // extern "C"
