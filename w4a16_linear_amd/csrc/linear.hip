// OPQ W4A16 linear layer: y = x W'^T (+ bias), with W' the bfloat16
// reconstruction of the stored weights (model card "OPQ INT4 Z-Image": the
// OPQLinear layer of the file list, decoded as in "技术细节 / 推理解码").
//
// W' is never written to HBM.  Each block builds the sixteen-entry table
// L_n[q] = bf16(G_q * m_n) of its weight rows, turns packed codes and sign
// bits into bfloat16 in registers (byte-plane lookups with v_perm), and feeds
// bf16 MFMA with fp32 accumulation.  The table holds the same values
// opq_dequantize writes; the scale is never applied after the product.
//
// Two paths:
//  * m <= kSkinnyMaxM: weight streaming, bound by HBM.  Blocks of 16 weight
//    rows x all of k, the waves of a block reducing in LDS (details below).
//  * otherwise: 256x256 output tiles with v_mfma_f32_32x32x16_bf16; x staged
//    through LDS (details below).
#include <algorithm>
#include <mutex>

#include "decode.hpp"
#include "device_common.hpp"
#include "group.hpp"

namespace opq {
namespace {

// ---------------------------------------------------------------- output

// Output element (row i of a 16-row weight fragment, column c of a 16-column x
// fragment) of v_mfma_f32_16x16x32_bf16 sits in lane 16 * (i / 4) + c,
// register i % 4.
// Outputs are written once and not read back by the kernel: nontemporal
// stores, as for the HBM-bound kernels (the tiled layer measures the same as
// with plain stores, within 0.5 %, when its inputs come from HBM).
__device__ __forceinline__ void store_y(void* y, bool y_bf16, int64_t at, float v) {
  if (y_bf16) __builtin_nontemporal_store((uint16_t)bf16_rne(v), static_cast<uint16_t*>(y) + at);
  else __builtin_nontemporal_store(v, static_cast<float*>(y) + at);
}

// ---------------------------------------------------------------- skinny path
//
// m <= 64: few flops per weight byte (2 m flops against 0.625 bytes), so the
// roofline is HBM; at these sizes the time goes to each wave's chain of k
// blocks and the launch rather than to the loads.  A block owns 16 weight
// rows (one fragment of
// v_mfma_f32_16x16x32_bf16, W' the A operand, x^T the B operand) and all of k;
// its waves (sixteen up to 32 x rows, eight above) take the 128-wide k blocks
// in turn and meet in LDS at the end, so no partial sums leave the block.
//
// Loads are laid out for the memory system, not for the MFMA: in a load, each
// group of four lanes reads 64 contiguous bytes (packed words: lane l reads
// part l%4 of weight row l/4; x: lane l reads 16-byte chunk l%16 of x row
// l/16 + 4i).  Packed words and sign words then move to the MFMA layout with
// ds_bpermute (lane (r, g) = (l%16, l/16) takes part g of row r), and x goes
// through a wave-private LDS stage, read back as B fragments.  Sub-step t of a
// k block contracts the 8-wide chunks {t, 4+t, 8+t, 12+t}: lane (r, g)
// supplies word t of part g, and chunk 4g + t of x.

constexpr int kSkinnyMaxM = 64;
constexpr int kSkRows = 16;                     // weight rows per block
constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * kWave;

// Waves per block of an instance.  Up to 32 x rows (one or two m blocks) a
// block runs 16 waves with one k block in flight per wave: twice the waves
// over the same 16 weight rows halve each wave's share of k, which hides more
// of the load latency than a second buffer did (m = 32 about 6% faster, m = 8
// and 16 4-7%).  The four-m-block instance has no registers or LDS to spare.
// The group-wise instances take it only with the block's tables prebuilt,
// which leaves them no per-k-block table build.
template <int NMB, int GS, bool kPre>
constexpr int sk_waves() { return (NMB <= 2 && (GS == 0 || kPre)) ? 16 : kSkWaves; }
constexpr int kSkBlockK = 128;                  // k per wave step
constexpr int kSkDepth = 2;                     // k blocks in flight per wave of an 8-wave block

// Element offset of 16-byte chunk c (0..15) of x row R in a wave's stage:
// 256-byte rows, chunks XOR-swizzled by the row so that the sixteen rows of a
// B fragment (same chunk) and the sixteen chunks of a row fall in different
// banks.
__device__ __forceinline__ int xs_off(int R, int c) { return R * kSkBlockK + ((c ^ (R & 15)) << 3); }

// GS > 0: the group-wise form (group.hpp).  With kPre (the block's 16 x k/GS
// groups are at most kSkPreGroups = 512) each of the first threads makes one group table at
// block start, straight from the levels and the stored max, into LDS as byte
// planes, group-major (a group's 16 rows adjacent, so a k block's reads hit 16
// consecutive 32-byte records); a k block then costs a lane two ds_read_b128.
// Otherwise the lane's table is rebuilt for every k block from the LDS
// significand table and the group max of its part.
constexpr int kSkPreGroups = kSkThreads;
template <int NMB, int GS, bool kPre = false>  // NMB: 16-row blocks of x (1, 2 or 4); GS: group or 0 (per row)
__global__ __launch_bounds__((sk_waves<NMB, GS, kPre>() * kWave)) void linear_skinny(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint32_t* __restrict__ sign, const float* __restrict__ scale,
    const uint16_t* __restrict__ scale16, const float* __restrict__ bias, int m, int n, int k,
    Levels lv, void* __restrict__ y, int y_bf16) {
  static_assert(GS == 0 || kPre || NMB <= 2, "the significand table and four x row blocks overfill LDS");
  static_assert(!kPre || GS > 0, "tables made at block start are for the group-wise form");
  // One k block per load batch, D batches in flight (a ring of register
  // buffers): batches of two k blocks took 14 % longer at m = 32 (more
  // registers, a later first MFMA).
  constexpr int CH = 1;
  constexpr int W = sk_waves<NMB, GS, kPre>();
  constexpr int D = W > kSkWaves ? 1 : (NMB >= 4 ? 2 : kSkDepth);
  constexpr int kXRows = 16 * NMB;
  constexpr int kXLoads = kXRows / 4;                   // x loads per lane per k block
  constexpr int kStage = kXRows * kSkBlockK;            // bf16 per wave stage
  constexpr int kOut = NMB * 4 * kWave;                 // outputs per wave, accumulator order
  static_assert(W * kOut * 4 <= W * kStage * 2, "reduction fits the stages");
  __shared__ __attribute__((aligned(16))) uint16_t s_x[W * kStage];
  __shared__ uint32_t s_lut[GS ? 1 : kSkRows][8];
  __shared__ __attribute__((aligned(16))) uint32_t s_mt[(GS && !kPre) ? kMantissas * 8 : 4];
  __shared__ __attribute__((aligned(16))) uint32_t s_glut[kPre ? kSkPreGroups * 8 : 4];
  float* s_red = reinterpret_cast<float*>(s_x);         // after the k loop

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n0 = blockIdx.x * kSkRows;
  const int kwords = k / 8, swords = k / 32;

  // This wave's k blocks: wave, wave + W, ...
  const int nkb = (k + kSkBlockK - 1) / kSkBlockK;
  const int mine = nkb > wave ? (nkb - 1 - wave) / W + 1 : 0;

  // Loader lanes.  Weight rows past n read row n - 1 and x rows past m read
  // row m - 1; neither is stored.
  const int lr = lane >> 2, lp = lane & 3;     // packed/sign: row lr, part lp
  const int xr = lane >> 4, xc = lane & 15;    // x: rows xr + 4i, chunk xc
  const int n0c = min(n0, n - 1);
  const char* pbase = reinterpret_cast<const char*>(packed + (int64_t)n0c * kwords);
  const char* sbase = reinterpret_cast<const char*>(sign + (int64_t)n0c * swords);
  const uint32_t rel = (uint32_t)(min(n0 + lr, n - 1) - n0c);
  const uint32_t p_off = rel * (uint32_t)kwords * 4u, s_off = rel * (uint32_t)swords * 4u;
  const char* xbase = reinterpret_cast<const char*>(x);
  uint32_t x_off[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) x_off[i] = (uint32_t)min(4 * i + xr, m - 1) * (uint32_t)k * 2u;

  // MFMA lanes: (r, g) takes its packed part from loader lane 4r + g.
  const int r = lane & 15, g = lane >> 4;
  const int src = (4 * r + g) * 4;

  uint4 wd[D][CH];
  uint32_t sw[D][CH];
  uint32_t hv[D][CH];  // GS > 0: float16 max of the lane's group in each k block
  uint4 xv[D][CH][kXLoads];
  const int ngroups = GS ? k / GS : 1;
  const uint16_t* hrow = GS ? scale16 + (int64_t)min(n0 + r, n - 1) * ngroups : nullptr;
  // Batch bi holds this wave's k blocks bi*CH .. bi*CH + CH - 1 (clamped to the
  // last).  In a final part block (k % 128 != 0) parts and chunks past k
  // re-read the block's first ones; the dequantizer zeroes those fragments.
  auto load_batch = [&](int bi, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int kb = (wave + W * min(bi * CH + j, mine - 1)) * kSkBlockK;
      const uint32_t kw = (uint32_t)(kb + 32 * lp < k ? kb + 32 * lp : kb);
      const uint32_t kx = (uint32_t)(kb + 8 * xc < k ? kb + 8 * xc : kb);
      wd[buf][j] = *reinterpret_cast<const uint4*>(pbase + p_off + kw / 2u);
      sw[buf][j] = *reinterpret_cast<const uint32_t*>(sbase + s_off + kw / 8u);
      if constexpr (GS > 0 && !kPre) hv[buf][j] = hrow[min((kb + 32 * g) / GS, ngroups - 1)];
#pragma unroll
      for (int i = 0; i < kXLoads; ++i)  // m <= 16: groups of 4 x rows wholly past m are skipped
        if (NMB > 1 || 4 * i < m) xv[buf][j][i] = *reinterpret_cast<const uint4*>(xbase + x_off[i] + kx * 2u);
    }
  };

  // The maxima the row tables are made from are requested ahead of the first
  // k blocks.  The compiler then waits for them before the batch goes out, so
  // only the four table waves issue their first batch a round trip late;
  // requested after the batch, they made the table build, and the barrier
  // after it, wait for the whole first batch (m <= 16: 7-9 % slower).
  const bool lut_lane = GS == 0 && wave < 4 && lane < kSkRows;
  const bool pre_lane = kPre && tid < kSkRows * ngroups;
  float mr = 0.0f;
  uint16_t m16_bits = 0;
  if (lut_lane) mr = scale[min(n0 + lane, n - 1)];
  if (pre_lane)
    m16_bits = scale16[(int64_t)min(n0 + (tid & (kSkRows - 1)), n - 1) * ngroups + tid / kSkRows];

  const int nbatch = (mine + CH - 1) / CH;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (nbatch > d) load_batch(d, d);

  // Byte planes of the block's 16 row tables: wave w < 4 makes entries
  // 4w .. 4w+3 of row `lane` (a wave-uniform code, so the levels stay in
  // scalar registers).
  if constexpr (GS > 0 && !kPre) build_mant_table(lv, s_mt);
  if (pre_lane) {
    // thread t: the table of group t / 16 of row n0 + t % 16 (all sixteen
    // entries, each with a compile-time level index)
    const RowLut t = make_row_lut(lv, f16_value(m16_bits));
    *reinterpret_cast<u32x4_t*>(&s_glut[8 * tid]) = u32x4_t{t.lo[0], t.lo[1], t.lo[2], t.lo[3]};
    *reinterpret_cast<u32x4_t*>(&s_glut[8 * tid + 4]) = u32x4_t{t.hi[0], t.hi[1], t.hi[2], t.hi[3]};
  }
  if (lut_lane) {
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t e = lut_entry(lv, 4 * wave + i, mr);
      lo |= (e & 0xFFu) << (8 * i);
      hi |= (e >> 8) << (8 * i);
    }
    s_lut[lane][wave] = lo;
    s_lut[lane][4 + wave] = hi;
  }
  // LDS writes done and visible; the loads stay in flight.
  lds_barrier();
  RowLut lut;
  if constexpr (GS == 0) {
    const uint4 lo = *reinterpret_cast<const uint4*>(&s_lut[r][0]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&s_lut[r][4]);
    lut.lo[0] = lo.x; lut.lo[1] = lo.y; lut.lo[2] = lo.z; lut.lo[3] = lo.w;
    lut.hi[0] = hi.x; lut.hi[1] = hi.y; lut.hi[2] = hi.z; lut.hi[3] = hi.w;
  }

  floatx4_t acc[NMB];
#pragma unroll
  for (int b = 0; b < NMB; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  uint16_t* stage = s_x + wave * kStage;
  auto compute_batch = [&](int bi, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int idx = bi * CH + j;
      if (idx < mine) {
        const int kb = (wave + W * idx) * kSkBlockK;
        const bool live = kb + 32 * g < k;
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
          // x rows past m only feed output columns that are never stored
          if (NMB == 1 && 4 * i >= m) continue;
          // element-wise: a whole-struct copy becomes a memcpy that keeps xv in scratch
          const uint4 v = xv[buf][j][i];
          *reinterpret_cast<u32x4_t*>(stage + xs_off(4 * i + xr, xc)) = u32x4_t{v.x, v.y, v.z, v.w};
        }
        const uint32_t words[4] = {
            (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)wd[buf][j].x),
            (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)wd[buf][j].y),
            (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)wd[buf][j].z),
            (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)wd[buf][j].w)};
        const uint32_t sb = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sw[buf][j]);
        if constexpr (kPre) {
          // (the launcher picks kPre only when 16 * ngroups <= kSkPreGroups)
          const int gidx = min(min((kb + 32 * g) / GS, ngroups - 1) * kSkRows + r, kSkPreGroups - 1);
          const uint4 lo = *reinterpret_cast<const uint4*>(&s_glut[8 * gidx]);
          const uint4 hi = *reinterpret_cast<const uint4*>(&s_glut[8 * gidx + 4]);
          lut.lo[0] = lo.x; lut.lo[1] = lo.y; lut.lo[2] = lo.z; lut.lo[3] = lo.w;
          lut.hi[0] = hi.x; lut.hi[1] = hi.y; lut.hi[2] = hi.z; lut.hi[3] = hi.w;
        } else if constexpr (GS > 0) {
          lut = group_lut(s_mt, hv[buf][j]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t o[4];
          decode_word_split(words[t], sb >> (8 * t), lut, o);
          if (!live) o[0] = o[1] = o[2] = o[3] = 0u;
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
          for (int b = 0; b < NMB; ++b) {
            const bf16x8_t bx = *reinterpret_cast<const bf16x8_t*>(stage + xs_off(16 * b + r, 4 * g + t));
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx, acc[b], 0, 0, 0);
          }
        }
      }
    }
  };

  for (int bi = 0; bi < nbatch; bi += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (bi + d < nbatch) {
        compute_batch(bi + d, d);
        if (bi + d + D < nbatch) load_batch(bi + d + D, d);
      }
    }
  }

  // Waves meet in LDS (the stages are free once every wave is here);
  // element o = (b * 4 + e) * 64 + lane.
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NMB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave * kOut + (b * 4 + e) * kWave + lane] = acc[b][e];
  __syncthreads();
  // Output (x row mm, weight row i): register i % 4 of lane 16 * (i / 4) + mm % 16
  // in block mm / 16; waves summed in a fixed order.
  for (int o = tid; o < kSkRows * kXRows; o += W * kWave) {
    const int i = o % kSkRows, mm = o / kSkRows;
    const int gcol = n0 + i;
    if (mm < m && gcol < n) {
      const int src_o = ((mm >> 4) * 4 + (i & 3)) * kWave + 16 * (i >> 2) + (mm & 15);
      float val = s_red[src_o];
#pragma unroll
      for (int w = 1; w < W; ++w) val += s_red[w * kOut + src_o];
      store_y(y, y_bf16, (int64_t)mm * n + gcol, val + (bias ? bias[gcol] : 0.0f));
    }
  }
}

// ---------------------------------------------------------------- tiled MFMA path
//
// Block tile 256 (x rows) x 256 (weight rows), k steps of 64,
// v_mfma_f32_32x32x16_bf16, eight waves (two per SIMD).  Wave w owns weight
// rows [32w, 32w + 32) of the tile (one B fragment per 16-wide k block) and all
// 256 x rows: 8 accumulators of 32x32 (128 fp32 per lane).
//
// Both operands reach LDS without passing through registers (buffer loads
// with the lds bit: lane i of a request writes 16 bytes, or 4, at the wave's
// LDS base + 16 i, from any offset it likes; the descriptor's range check
// returns zeros past the operand):
//  * x: NXS stages of 256 rows x 64 k (32 KB).  Row r is 128 bytes; its 16-byte
//    chunk c (k order) sits at chunk c ^ ((r >> 1) & 7), which keeps the
//    fragment reads below free of bank conflicts.  The lane that fills a slot
//    fetches the chunk that belongs there, so the four lanes of a quad still
//    read 64 contiguous bytes of one row.
//  * weights: NWS stages of a step pair (128 k): the 64 code bytes of each of
//    the 256 rows (16-byte chunk c of row r at chunk c ^ ((r >> 2) & 3)), then
//    each row's four sign words.
// A lane's offsets are fixed for the whole tile; the step's part goes in the
// scalar offset.
//
// Each weight row is decoded once per tile, in registers: lane (r, h) of wave w
// (row 32w + r, half h of the step) takes the four code words of k
// 64 kt + 32 h ... + 31 and turns word s into the eight bf16 values of sub-step
// s with its row's table held as byte planes (v_perm lookups, k order), so
// sub-step s contracts the 8-wide k blocks {s, 4 + s}; the x fragments are read
// for the same blocks.
//
// Pipeline, one barrier per k step:
//  * x of step kt + NXS - 1 is requested in step kt, after the barrier that
//    ends step kt - 1 (its stage last served step kt - 1), and waited for
//    (vmcnt) before the barrier that ends step kt + NXS - 2, which publishes it;
//  * the weights of pair q are requested in step 2q + 1 - 2 NWS (their stage
//    last served pair q - NWS) and are complete long before their first use;
//  * the code words and the first decode of step kt + 1 are done before the
//    barrier that ends step kt (their pair was published steps earlier), so after
//    the barrier a wave only waits for its first x fragments.
// Requests past the last step read whatever lies there (never used), which keeps
// the wait counts static.  A final half step (k % 64 = 32) zeroes the dead half
// of the weight fragment; its x slots re-read the step's first half.
//
// Within a sub-step each MFMA is followed by one x fragment read of the next
// sub-step and a share of the decode (and, in sub-steps 1 and 2, of the step's
// requests; in sub-step 0 with two x stages): the decode's VALU work then runs
// while the wave's own MFMAs execute instead of alternating with them.  Each stage is an LDS array of its
// own and the main loop is unrolled over the stages' common period, so every
// access names its stage at compile time; the compiler then tells a read of one
// stage from the loads in flight to another and inserts no wait for them.  The
// barrier is the one for direct-to-LDS kernels (lds_barrier_dma): a workgroup
// release fence on LDS would wait for every load in flight.
//
// GS > 0: the group-wise form (group.hpp).  The lane's table is rebuilt from the
// LDS significand table when its group changes; the float16 group maxima are
// loaded two steps ahead.  That table takes 32 KB of LDS, so these instances run
// two x stages and two weight stages.

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kTVALUPerMFMA = 4;  // VALU slots after each MFMA in the forced interleave
constexpr int kTThreads = 512;
constexpr int kXStageBytes = kTM * kTK * 2;        // 32 KB
constexpr int kWCodeBytes = kTN * 64;              // codes of a step pair, 16 KB
constexpr int kWStageBytes = kWCodeBytes + kTN * 16;  // + four sign words per row, 20 KB
constexpr int kXLoads = kXStageBytes / 1024 / (kTThreads / kWave);     // 4 per wave per step
constexpr int kWCodeLoads = kWCodeBytes / 1024 / (kTThreads / kWave);  // 2 per wave per pair
constexpr int kWSignLoads = kTN * 16 / 256 / (kTThreads / kWave);      // 2 per wave per pair
constexpr int kWLoads = kWCodeLoads + kWSignLoads;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Fourth word of a raw buffer descriptor: 32-bit data format, no swizzle or stride.
constexpr int kBufferFlags = 0x00020000;

// LDS byte offset of 16-byte chunk c of x row r within a stage.
__device__ __forceinline__ uint32_t x_slot(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

// A step's position in the unrolled main loop (its stages are then known at
// compile time), or kDynamic: stages chosen at run time.
template <int I> struct StepPos { static constexpr int value = I; };
constexpr int kDynamic = -1;

template <int U, typename F>
__device__ __forceinline__ void unroll_steps(F&& f) {
  if constexpr (U > 0) {
    unroll_steps<U - 1>(f);
    f(StepPos<U - 1>{});
  }
}

template <int GS> constexpr int tiled_x_stages() { return GS ? 2 : 3; }
template <int GS> constexpr int tiled_w_stages() { return GS ? 2 : 3; }
template <int GS>
constexpr int tiled_lds_bytes() {
  return tiled_x_stages<GS>() * kXStageBytes + tiled_w_stages<GS>() * kWStageBytes +
         (GS ? kMantissas * 32 : 0);
}
static_assert(tiled_lds_bytes<0>() <= 160 * 1024 && tiled_lds_bytes<32>() <= 160 * 1024,
              "the stages fit the 160 KB of LDS");

// s_waitcnt vmcnt(N) for N < 64, every other counter left open.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// kSplit: block b takes tile b % T (T tiles) and the k steps [s0, s0 +
// slice_steps) of slice b / T (s0 = slice * slice_steps, an even step, so
// weight pairs stay whole), and writes its float32 sums without the bias to
// plane `slice` of `part` ([S][m][n]); linear_split_reduce then adds the
// planes in slice order.  Taken when the tiles alone would leave most CUs idle.
template <bool kHalfTail, int GS, bool kSplit = false>
__global__ __launch_bounds__(kTThreads, 1) void linear_tiled(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint32_t* __restrict__ sign, const float* __restrict__ scale,
    const uint16_t* __restrict__ scale16, const float* __restrict__ bias, int m, int n, int k,
    int tiles_m, Levels lv, void* __restrict__ y, int y_bf16, int slice_steps,
    float* __restrict__ part) {
  static_assert(!(kSplit && (kHalfTail || GS > 0)), "split-k: per-row scales, k a multiple of 64");
  constexpr int NXS = tiled_x_stages<GS>(), NWS = tiled_w_stages<GS>();
  constexpr int LX = NXS - 1;  // x of step kt + LX is requested in step kt
  // One array per stage: with the stage of every access known at compile time
  // the compiler can tell an LDS read from the direct-to-LDS writes in flight
  // to other stages, and does not wait for them.
  __shared__ __attribute__((aligned(1024))) uint8_t s_x0[kXStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x1[kXStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x2[NXS > 2 ? kXStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w0[kWStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w1[kWStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w2[NWS > 2 ? kWStageBytes : 16];
  __shared__ __attribute__((aligned(16))) uint32_t s_mt[GS ? kMantissas * 8 : 4];
  auto x_stage = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return i == 0 ? s_x0 : (i == 1 ? s_x1 : s_x2);
  };
  auto w_stage = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return i == 0 ? s_w0 : (i == 1 ? s_w1 : s_w2);
  };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // uniform across the wave: the LDS destinations of the loads are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ntiles = tiles_m * ((n + kTN - 1) / kTN);
  const int tile = kSplit ? (int)(blockIdx.x % (unsigned)ntiles) : (int)blockIdx.x;
  const int slice = kSplit ? (int)(blockIdx.x / (unsigned)ntiles) : 0;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int m0 = tile_m * kTM;
  const int n0 = tile_n * kTN;
  const int h = lane >> 5;                         // which half of the k step
  const int rr = wave * 32 + (lane & 31);          // this lane's weight row in the tile
  const int brow = n0 + rr;
  const int kwords = k / 8, swords = k / 32;
  const int all_steps = (k + kTK - 1) / kTK;
  const int s0 = kSplit ? slice * slice_steps : 0;  // first k step of this block
  const int nsteps = kSplit ? min(slice_steps, all_steps - s0) : all_steps;

  // ---- loads.  x: load i of wave w fills 1 KB block 4w + i of a stage, i.e.
  // rows 8(4w + i) .. + 7; lane l the slot (row 8(4w + i) + l/8, chunk l%8).
  const char* xbase = reinterpret_cast<const char*>(x + (int64_t)m0 * k);
  uint32_t x_off[kXLoads];   // byte offset of the lane's chunk, step 0
  int x_chunk[kXLoads];      // its chunk (k / 8 within the step)
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int r = 8 * (kXLoads * wave + i) + (lane >> 3);
    x_chunk[i] = (lane & 7) ^ ((r >> 1) & 7);
    const uint32_t rowc = (uint32_t)(min(m0 + r, m - 1) - m0);
    x_off[i] = rowc * (uint32_t)k * 2u + (uint32_t)x_chunk[i] * 16u;
  }
  // The requests go through buffer descriptors (base and size in scalar
  // registers, a 32-bit offset per lane), whose range check turns any offset
  // past the end into zeros; offsets stay below 2^31 (a tile's rows).
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xbase, (short)0, (int)min((int64_t)(m - m0) * k * 2, (int64_t)0x7FFFFFFF), kBufferFlags);
  // The step's offset goes in the scalar offset; requests for steps past the
  // last read whatever lies there (never used).  In a final half step the
  // chunks past k re-read the step's first half, so only values of the same x
  // row ever meet the zeroed half of the weight fragment.
  auto load_x = [&](int kt, uint8_t* st) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)(kt + s0) * (kTK * 2);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      uint32_t off = x_off[i];
      if constexpr (kHalfTail) {
        if (kt == nsteps - 1 && x_chunk[i] >= 4) off -= 64u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lds_ptr_t)(st + (kXLoads * wave + i) * 1024),
                                               16, off, soff, 0, 0);
    }
  };
  // weights of pair q: code load i of wave w fills 1 KB block 2w + i of the code
  // region (rows 16(2w + i) + l/4, chunk slot l%4); sign load i fills 256 B block
  // 2w + i (rows 16(2w + i) + l/4, word l%4).
  const int n0c = min(n0, n - 1);
  const char* pbase = reinterpret_cast<const char*>(packed + (int64_t)n0c * kwords);
  const char* sbase = reinterpret_cast<const char*>(sign + (int64_t)n0c * swords);
  // byte offsets of the lane's code chunk and sign word in pair 0
  uint32_t wc_off[kWCodeLoads], ws_off[kWSignLoads];
#pragma unroll
  for (int i = 0; i < kWCodeLoads; ++i) {
    const int r = 16 * (kWCodeLoads * wave + i) + (lane >> 2);
    wc_off[i] = (uint32_t)(min(n0 + r, n - 1) - n0c) * (uint32_t)kwords * 4u +
                (uint32_t)((lane & 3) ^ ((r >> 2) & 3)) * 16u;
  }
#pragma unroll
  for (int i = 0; i < kWSignLoads; ++i) {
    const int r = 16 * (kWSignLoads * wave + i) + (lane >> 2);
    ws_off[i] = (uint32_t)(min(n0 + r, n - 1) - n0c) * (uint32_t)swords * 4u + (uint32_t)(lane & 3) * 4u;
  }
  const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)pbase, (short)0, (int)min((int64_t)(n - n0c) * kwords * 4, (int64_t)0x7FFFFFFF), kBufferFlags);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)sbase, (short)0, (int)min((int64_t)(n - n0c) * swords * 4, (int64_t)0x7FFFFFFF), kBufferFlags);
  auto load_w = [&](int q, uint8_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kWCodeLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p_rsrc, (lds_ptr_t)(st + (kWCodeLoads * wave + i) * 1024),
                                               16, wc_off[i], (uint32_t)(q + s0 / 2) * 64u, 0, 0);
#pragma unroll
    for (int i = 0; i < kWSignLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          s_rsrc, (lds_ptr_t)(st + kWCodeBytes + (kWSignLoads * wave + i) * 256), 4, ws_off[i],
          (uint32_t)(q + s0 / 2) * 16u, 0, 0);
  };

  // ---- the lane's table and code words.
  RowLut lut;
  if constexpr (GS == 0) lut = make_row_lut(lv, scale[min(brow, n - 1)]);
  const int ngroups = GS ? k / GS : 1;
  const uint16_t* hrow = GS ? scale16 + (int64_t)min(brow, n - 1) * ngroups : nullptr;
  auto load_h = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    if constexpr (GS > 0)
      return hrow[min((min(kt, nsteps - 1) * kTK + 32 * h) / GS, ngroups - 1)];
    else
      return 0u;
  };
  uint32_t h_next = 0u, h_load = 0u;  // GS > 0: maxima of steps kt + 1 and kt + 2

  // codes (4 words) and sign word of step kt for this lane
  const uint32_t wr_code = (uint32_t)rr * 64u, wr_sign = (uint32_t)kWCodeBytes + (uint32_t)rr * 16u;
  const uint32_t wr_swz = (uint32_t)((rr >> 2) & 3);
  auto read_w = [&](int kt, const uint8_t* st, uint4& pw, uint32_t& sw) __attribute__((always_inline)) {
    const uint32_t c = (uint32_t)(2 * (kt & 1) + h);
    pw = *reinterpret_cast<const uint4*>(st + wr_code + ((c ^ wr_swz) << 4));
    sw = *reinterpret_cast<const uint32_t*>(st + wr_sign + c * 4u);
  };
  auto decode_b = [&](int kt, int s, const uint4& pwv, uint32_t swv, bf16x8_t& b)
      __attribute__((always_inline)) {
    const uint32_t words[4] = {pwv.x, pwv.y, pwv.z, pwv.w};
    uint32_t o[4];
    decode_word_split(words[s], swv >> (8 * s), lut, o);
    if constexpr (kHalfTail) {
      if (kt == nsteps - 1 && h == 1) o[0] = o[1] = o[2] = o[3] = 0u;
    }
    b = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  };
  // x fragments of sub-step s of step kt: rows 32 mi + (lane & 31), chunk s + 4h
  auto read_a = [&](const uint8_t* st, int s, bf16x8_t (&a)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      const int r = mi * 32 + (lane & 31);
      a[mi] = *reinterpret_cast<const bf16x8_t*>(st + x_slot(r, s + 4 * h));
    }
  };

  floatx16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

  uint4 pw;
  uint32_t sw;
  // Two B fragments: the next sub-step's decode fills one while this
  // sub-step's MFMAs read the other, so it can run between them.
  bf16x8_t a_frag[8], b_buf[2];
  if (nsteps > 0) {
    // prologue: x of steps 0 .. LX - 1, weight pairs 0 .. NWS - 1
    uint32_t h0 = 0u;
    if constexpr (GS > 0) {
      h0 = load_h(0);
      h_next = load_h(1);
    }
#pragma unroll
    for (int j = 0; j < LX; ++j) load_x(j, x_stage(j));
#pragma unroll
    for (int q = 0; q < NWS; ++q) load_w(q, w_stage(q));
    if constexpr (GS > 0) build_mant_table(lv, s_mt);
    wait_vm<0>();
    lds_barrier_dma();
    if constexpr (GS > 0) lut = group_lut(s_mt, h0);
    read_w(0, s_w0, pw, sw);
    decode_b(0, 0, pw, sw, b_buf[0]);
    read_a(s_x0, 0, a_frag);
  }

  // One k step.  pos: StepPos<u> for the u-th step of an unrolled group of kUnroll
  // (kt % kUnroll == u, every stage a compile-time choice), or StepPos<kDynamic>.
  constexpr int kUnroll = NXS * 2 * NWS / (NXS == NWS ? NXS : 1);  // lcm(NXS, 2 NWS)
  static_assert(kUnroll % NXS == 0 && kUnroll % (2 * NWS) == 0, "stage periods divide the unroll");
  auto step = [&](int kt, auto pos) __attribute__((always_inline)) {
    constexpr int u = decltype(pos)::value;
    const bool odd = u >= 0 ? (u & 1) : (kt & 1);
    // stage of x of step kt + j, and of the weight pair holding step kt + j
    auto xs = [&](int j) __attribute__((always_inline)) {
      return x_stage(u >= 0 ? (u + j) % NXS : (kt + j) % NXS);
    };
    auto ws = [&](int j) __attribute__((always_inline)) {
      return w_stage(u >= 0 ? ((u + j) / 2) % NWS : ((kt + j) / 2) % NWS);
    };
    // requests after the barrier that ended step kt - 1: the group max of step
    // kt + 2 first (a plain load, waited for by the compiler where it is used),
    // then x of step kt + LX, then (odd steps) the weights of pair
    // (kt - 1) / 2 + NWS, into the stage of pair (kt - 1) / 2
    if constexpr (GS > 0) h_load = load_h(kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    // With three x stages the step's requests go out in sub-steps 1 (x) and
    // 2 (weights), one after every other MFMA, rather than in a burst at the
    // start of the step, when all eight waves leave the barrier together
    // (about 1 % faster on all three DiT shapes; the order of the requests,
    // and so the wait counts below, are unchanged).  With two x stages the x
    // of step kt + 1 must land within step kt: requested at its start.
    constexpr bool kSpread = LX == 2;
    if constexpr (!kSpread) {
      load_x(kt + LX, xs(LX));
      if (odd) load_w((kt - 1) / 2 + NWS, ws(-1));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      if constexpr (kSpread) {
        if (s == 1) load_x(kt + LX, xs(LX));
        if (s == 2 && odd) load_w((kt - 1) / 2 + NWS, ws(-1));
      }
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag[mi], b_buf[cur], acc[mi], 0, 0, 0);
      if (s < 3) {
        read_a(xs(0), s + 1, a_frag);
        decode_b(kt, s + 1, pw, sw, b_buf[nxt]);
        // Interleave: after each MFMA, one x fragment read of the next sub-step
        // (its register is free once that MFMA has issued), a share of the
        // decode and one of this step's load requests (sub-steps 1 and 2, after
        // every other MFMA; with two x stages, sub-step 0), so the VALU work
        // runs while this wave's MFMAs execute.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          if (kSpread ? ((s == 1 || s == 2) && (i & 1)) : s == 0)
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
          __builtin_amdgcn_sched_group_barrier(0x002, kTVALUPerMFMA, 0);  // VALU
        }
      } else {
        // the next step's code words (their pair is published) and first decode
        read_w(kt + 1, ws(1), pw, sw);
        if constexpr (GS > 0) {
          // the table of step kt + 1, when it starts a new group (every step
          // for groups of 32 and 64: the two halves of a step differ or the
          // group is one step long)
          if (GS <= kTK || ((kt + 1) * kTK) % GS == 0) lut = group_lut(s_mt, h_next);
          h_next = h_load;
        }
        decode_b(kt + 1, 0, pw, sw, b_buf[nxt]);
        // the next step's code words first, then the decode between the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kTVALUPerMFMA, 0);  // VALU
        }
        // x of step kt + 1 is complete: every request issued before it is done.
        // Issued after it: with three x stages, the x of step kt + 2 and one
        // pair of weights; with two, the weights of this step (odd steps).
        if constexpr (LX == 2) {
          wait_vm<kXLoads + kWLoads>();
        } else {
          if (odd) wait_vm<kWLoads>();
          else wait_vm<0>();
        }
        lds_barrier_dma();
        read_a(xs(1), 0, a_frag);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // steps are not interleaved: that costs registers
  };
  int kt = 0;
  for (; kt + kUnroll <= nsteps; kt += kUnroll)
    unroll_steps<kUnroll>([&](auto pos) __attribute__((always_inline)) {
      step(kt + decltype(pos)::value, pos);
    });
  for (; kt < nsteps; ++kt) step(kt, StepPos<kDynamic>{});
  wait_vm<0>();  // no load may still be writing LDS when the block ends

  // 32x32 accumulator layout: register e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.  Whole tiles store without a bound check (nontemporal, as
  // store_y).
  // split-k: float32 sums of this slice, no bias, into its plane of `part`
  void* yo = kSplit ? static_cast<void*>(part + (int64_t)slice * m * n) : y;
  const int ybf = kSplit ? 0 : y_bf16;
  const float bv = (!kSplit && bias && brow < n) ? bias[brow] : 0.0f;
  const bool whole = m0 + kTM <= m && n0 + kTN <= n;
  if (whole && !ybf) {
    float* yrow = static_cast<float*>(yo) + (int64_t)(m0 + 4 * h) * n + brow;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        __builtin_nontemporal_store(acc[mi][e] + bv, yrow + (int64_t)(mi * 32 + 8 * (e >> 2) + (e & 3)) * n);
  } else if (whole) {
    uint16_t* yrow = static_cast<uint16_t*>(yo) + (int64_t)(m0 + 4 * h) * n + brow;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        __builtin_nontemporal_store((uint16_t)bf16_rne(acc[mi][e] + bv),
                                    yrow + (int64_t)(mi * 32 + 8 * (e >> 2) + (e & 3)) * n);
  } else {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + mi * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < m && brow < n) store_y(yo, ybf, (int64_t)row * n + brow, acc[mi][e] + bv);
      }
  }
}

// ---------------------------------------------------------------- dense bf16 weights
//
// y = x W'^T with W' already bfloat16 in memory ([n][k]).  This serves the
// other code widths: opq_linear_bits first writes W' into a workspace with the
// b-bit dequantizer, the way the card's OPQLinear decodes its weights before a
// dense matmul.  The kernels are the two above with the weight operand read
// instead of decoded.
//
// Tiled (m > 64): linear_tiled's tile, waves and fragments, with W' staged like
// x (256 rows x 64 k per stage, same swizzle, buffer loads straight to LDS),
// two stages of each.  A wave's B fragment is one ds_read_b128 per sub-step.

template <bool kHalfTail>
__global__ __launch_bounds__(kTThreads, 1) void linear_dense_tiled(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd, const float* __restrict__ bias,
    int m, int n, int k, int tiles_m, void* __restrict__ y, int y_bf16) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_x0[kXStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x1[kXStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w0[kXStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w1[kXStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int m0 = tile_m * kTM;
  const int n0 = tile_n * kTN;
  const int h = lane >> 5;
  const int brow = n0 + wave * 32 + (lane & 31);
  const int nsteps = (k + kTK - 1) / kTK;

  // both operands: load i of wave w fills 1 KB block 4w + i of a stage (rows
  // 8(4w + i) + l/8, chunk slot l%8), as in linear_tiled
  const char* xbase = reinterpret_cast<const char*>(x + (int64_t)m0 * k);
  const char* wbase = reinterpret_cast<const char*>(wd + (int64_t)n0 * k);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xbase, (short)0, (int)min((int64_t)(m - m0) * k * 2, (int64_t)0x7FFFFFFF), kBufferFlags);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wbase, (short)0, (int)min((int64_t)(n - n0) * k * 2, (int64_t)0x7FFFFFFF), kBufferFlags);
  uint32_t x_off[kXLoads], w_off[kXLoads];
  int chunk[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int r = 8 * (kXLoads * wave + i) + (lane >> 3);
    chunk[i] = (lane & 7) ^ ((r >> 1) & 7);
    x_off[i] = (uint32_t)(min(m0 + r, m - 1) - m0) * (uint32_t)k * 2u + (uint32_t)chunk[i] * 16u;
    w_off[i] = (uint32_t)(min(n0 + r, n - 1) - n0) * (uint32_t)k * 2u + (uint32_t)chunk[i] * 16u;
  }
  auto load = [&](int kt, uint8_t* sx, uint8_t* sw) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)kt * (kTK * 2);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      uint32_t xo = x_off[i], wo = w_off[i];
      if constexpr (kHalfTail) {
        // chunks past k in the final half step re-read the step's first half
        if (kt == nsteps - 1 && chunk[i] >= 4) { xo -= 64u; wo -= 64u; }
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lds_ptr_t)(sx + (kXLoads * wave + i) * 1024),
                                               16, xo, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_ptr_t)(sw + (kXLoads * wave + i) * 1024),
                                               16, wo, soff, 0, 0);
    }
  };
  auto read_a = [&](const uint8_t* st, int s, bf16x8_t (&a)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
      a[mi] = *reinterpret_cast<const bf16x8_t*>(st + x_slot(mi * 32 + (lane & 31), s + 4 * h));
  };
  auto read_b = [&](const uint8_t* st, int kt, int s, bf16x8_t& b) __attribute__((always_inline)) {
    b = *reinterpret_cast<const bf16x8_t*>(st + x_slot(wave * 32 + (lane & 31), s + 4 * h));
    if constexpr (kHalfTail) {
      if (kt == nsteps - 1 && h == 1) b = bf16x8_t{};  // the dead half of the final half step
    }
  };

  floatx16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
  bf16x8_t a_frag[8], b_buf[2];
  if (nsteps > 0) {
    load(0, s_x0, s_w0);
    wait_vm<0>();
    lds_barrier_dma();
    read_a(s_x0, 0, a_frag);
    read_b(s_w0, 0, 0, b_buf[0]);
  }
  // step kt: stage kt & 1; the loads of step kt + 1 go to the other stage, which
  // served step kt - 1, and are waited for before this step's barrier
  auto step = [&](int kt, auto par) __attribute__((always_inline)) {
    constexpr int p = decltype(par)::value;
    uint8_t* sx = p ? s_x1 : s_x0;
    uint8_t* sw = p ? s_w1 : s_w0;
    uint8_t* nx = p ? s_x0 : s_x1;
    uint8_t* nw = p ? s_w0 : s_w1;
    load(kt + 1, nx, nw);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag[mi], b_buf[cur], acc[mi], 0, 0, 0);
      if (s < 3) {
        read_a(sx, s + 1, a_frag);
        read_b(sw, kt, s + 1, b_buf[nxt]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          if (s == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
        }
      } else {
        wait_vm<0>();
        lds_barrier_dma();
        read_a(nx, 0, a_frag);
        read_b(nw, kt + 1, 0, b_buf[nxt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + 1 < nsteps; kt += 2) {
    step(kt, StepPos<0>{});
    step(kt + 1, StepPos<1>{});
  }
  if (kt < nsteps) step(kt, StepPos<0>{});
  wait_vm<0>();  // no load may still be writing LDS when the block ends

  const float bv = (bias && brow < n) ? bias[brow] : 0.0f;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + mi * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (row < m && brow < n) store_y(y, y_bf16, (int64_t)row * n + brow, acc[mi][e] + bv);
    }
}

// Skinny (m <= 64): linear_skinny's blocks (16 weight rows, all of k, waves
// over 128-wide k blocks, a reduction in LDS) with lane (r, g) reading the 64
// bytes of W' row r, k 32 g ... + 31 of each k block straight into its four A
// fragments.
template <int NMB>  // 16-row blocks of x (1, 2 or 4)
__global__ __launch_bounds__((NMB <= 2 ? 16 : 8) * kWave) void linear_dense_skinny(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd, const float* __restrict__ bias,
    int m, int n, int k, void* __restrict__ y, int y_bf16) {
  constexpr int W = NMB <= 2 ? 16 : 8;
  constexpr int kXRows = 16 * NMB;
  constexpr int kXL = kXRows / 4;                   // x loads per lane per k block
  constexpr int kStage = kXRows * kSkBlockK;
  constexpr int kOut = NMB * 4 * kWave;
  __shared__ __attribute__((aligned(16))) uint16_t s_x[W * kStage];
  float* s_red = reinterpret_cast<float*>(s_x);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n0 = blockIdx.x * kSkRows;
  const int nkb = (k + kSkBlockK - 1) / kSkBlockK;
  const int mine = nkb > wave ? (nkb - 1 - wave) / W + 1 : 0;
  const int xr = lane >> 4, xc = lane & 15;
  const int r = lane & 15, g = lane >> 4;
  const char* wrow = reinterpret_cast<const char*>(wd + (int64_t)min(n0 + r, n - 1) * k);
  const char* xbase = reinterpret_cast<const char*>(x);
  uint32_t x_off[kXL];
#pragma unroll
  for (int i = 0; i < kXL; ++i) x_off[i] = (uint32_t)min(4 * i + xr, m - 1) * (uint32_t)k * 2u;

  floatx4_t acc[NMB];
#pragma unroll
  for (int b = 0; b < NMB; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* stage = s_x + wave * kStage;
  for (int idx = 0; idx < mine; ++idx) {
    const int kb = (wave + W * idx) * kSkBlockK;
    const bool live = kb + 32 * g < k;
    const int kw = live ? kb + 32 * g : kb;          // a part past k re-reads the first
    uint4 wv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wv[t] = *reinterpret_cast<const uint4*>(wrow + (int64_t)(kw + 8 * t) * 2);
    const int kx = kb + 8 * xc < k ? kb + 8 * xc : kb;
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
      if (NMB == 1 && 4 * i >= m) continue;          // x rows wholly past m
      const uint4 v = *reinterpret_cast<const uint4*>(xbase + x_off[i] + (uint32_t)kx * 2u);
      *reinterpret_cast<u32x4_t*>(stage + xs_off(4 * i + xr, xc)) = u32x4_t{v.x, v.y, v.z, v.w};
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 a4 = live ? wv[t] : make_uint4(0u, 0u, 0u, 0u);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, a4);
#pragma unroll
      for (int b = 0; b < NMB; ++b) {
        const bf16x8_t bx = *reinterpret_cast<const bf16x8_t*>(stage + xs_off(16 * b + r, 4 * g + t));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx, acc[b], 0, 0, 0);
      }
    }
    wave_lds_sync();  // the stage is rewritten by the next k block
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NMB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave * kOut + (b * 4 + e) * kWave + lane] = acc[b][e];
  __syncthreads();
  for (int o = tid; o < kSkRows * kXRows; o += W * kWave) {
    const int i = o % kSkRows, mm = o / kSkRows;
    const int gcol = n0 + i;
    if (mm < m && gcol < n) {
      const int src_o = ((mm >> 4) * 4 + (i & 3)) * kWave + 16 * (i >> 2) + (mm & 15);
      float val = s_red[src_o];
#pragma unroll
      for (int w = 1; w < W; ++w) val += s_red[w * kOut + src_o];
      store_y(y, y_bf16, (int64_t)mm * n + gcol, val + (bias ? bias[gcol] : 0.0f));
    }
  }
}

}  // namespace

namespace {

// y[mm][c] = sum over s = 0 .. S-1 of part[s][mm][c], in that order, + bias[c]
// (the split-k planes of linear_tiled).
__global__ __launch_bounds__(256) void linear_split_reduce(const float* __restrict__ part,
                                                           int nslice, int64_t count, int n,
                                                           const float* __restrict__ bias,
                                                           void* __restrict__ y, int y_bf16) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * 256) {
    float v = part[e];
    for (int s = 1; s < nslice; ++s) v += part[(int64_t)s * count + e];
    store_y(y, y_bf16, e, v + (bias ? bias[e % n] : 0.0f));
  }
}

constexpr int64_t kPartCUs = 256;                        // the part's CUs
constexpr int64_t kMaxSplitBytes = int64_t(128) << 20;   // largest partial-sum workspace

// Split-k of the tiled layer (per-row scales, k a multiple of 64): when its
// tiles would cover at most a quarter of the CUs, S slices of an even number
// of k steps each, so that about kPartCUs blocks run, each at least 8 steps
// long.  Returns S (1: no split) and the steps per slice.  Measured against
// the unsplit grid (or the x-row slices where the call took them), one box,
// graph replay: n = k = 3840 at m = 256 / 512 / 1024 54 / 71 / 74 -> 32 / 45 /
// 61 us, 1024 x 3840 x 10240 181 -> 110 us, 130 x 1024 x 8192 48 -> 27 us,
// 512 x 1024 x 8192 152 -> 34 us.  Not taken for m <= 128 (the x-row slices
// are faster: m = 65 20 against 28 us) or for more than 64 tiles (m = 2048,
// n = 3840: 87 unsplit against 91 us).
int tiled_split(int64_t m, int64_t n, int64_t k, int* slice_steps) {
  if (m <= 2 * kSkinnyMaxM || n < 1 || k % kTK) return 1;
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  const int64_t steps = k / kTK;
  if (tiles * 4 > kPartCUs) return 1;
  int64_t s = std::min(kPartCUs / tiles, steps / 8);
  if (s < 2) return 1;
  int64_t sps = (steps + s - 1) / s;
  sps += sps & 1;
  s = (steps + sps - 1) / sps;
  if (s < 2 || s * m * n * 4 > kMaxSplitBytes) return 1;
  if (slice_steps) *slice_steps = (int)sps;
  return (int)s;
}

// Mid-size m (a few 256-row tiles): the tiled kernel's grid then covers few
// CUs while each tile still walks all of k, and slices of up to 64 x rows
// through the skinny kernel (each slice streaming the whole weight once) can
// finish first.  Rough costs on this part, in microseconds, fitted to
// measurements at n = 3840..20480, k = 3840..10240, m = 65..512 (both sides
// within ~10 % at the crossover): a k step of a grid of at most one tile per
// CU takes ~1.25; a slice ~3 plus ~0.75 per million weights.  For example 3840 x
// 3840 weights at m = 128 take 27 us as two slices against 76 us tiled, and
// 20480 x 3840 at m = 65 stay tiled (76 against 82 us).  Both paths are exact
// to the same tolerance; only the order of the k sum differs.
bool mid_m_as_slices(int64_t m, int64_t n, int64_t k, bool split_ok = false) {
  if (m <= kSkinnyMaxM) return false;
  const int64_t cus = kPartCUs;  // a function of the shape alone
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  const int64_t waves = (tiles + cus - 1) / cus;
  double tiled_us = (double)waves * (double)((k + kTK - 1) / kTK) * 1.25;
  int sps = 0;
  const int split = split_ok ? tiled_split(m, n, k, &sps) : 1;
  if (split > 1)  // a slice's steps, plus the reduce: a launch and the planes' bytes
    tiled_us = sps * 1.25 + 12.0 + (double)split * m * n * 8 / 4e6;
  const double slices = (double)((m + kSkinnyMaxM - 1) / kSkinnyMaxM);
  const double sliced_us = slices * (3.0 + 0.75e-3 * (double)n * (double)k / 1000.0);
  return sliced_us < tiled_us;
}

template <int GS>
hipError_t launch_linear_any(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                             const float* scale, const uint16_t* scale16, const float* bias,
                             int64_t m, int64_t n, int64_t k, const Levels& lv, void* y,
                             bool y_bf16, float* part, hipStream_t stream) {
  if (mid_m_as_slices(m, n, k, GS == 0)) {
    const int64_t ybytes = y_bf16 ? 2 : 4;
    for (int64_t r = 0; r < m; r += kSkinnyMaxM) {
      const int64_t mm = m - r < kSkinnyMaxM ? m - r : kSkinnyMaxM;
      const hipError_t e = launch_linear_any<GS>(x + r * k, packed, sign, scale, scale16, bias, mm,
                                                 n, k, lv, static_cast<char*>(y) + r * n * ybytes,
                                                 y_bf16, part, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (m <= kSkinnyMaxM) {
    const int64_t blocks = (n + kSkRows - 1) / kSkRows;
    // group tables made at block start when the block's groups fit
    const bool pre = GS > 0 && kSkRows * (k / (GS ? GS : 1)) <= kSkPreGroups;
    auto k2 = pre ? linear_skinny<2, GS, (GS > 0)> : linear_skinny<2, GS>;
    const unsigned t2 = (unsigned)(pre ? sk_waves<2, GS, (GS > 0)>() : sk_waves<2, GS, false>()) * kWave;
    if (GS > 0 && !pre && m > 32) {
      // The significand table leaves no room for four x row blocks: two
      // launches of up to 32 x rows each.
      hipLaunchKernelGGL(k2, dim3((unsigned)blocks), dim3(t2), 0, stream, x, packed,
                         sign, scale, scale16, bias, 32, (int)n, (int)k, lv, y, (int)y_bf16);
      const int64_t ybytes = y_bf16 ? 2 : 4;
      hipLaunchKernelGGL(k2, dim3((unsigned)blocks), dim3(t2), 0, stream, x + 32 * k,
                         packed, sign, scale, scale16, bias, (int)(m - 32), (int)n, (int)k, lv,
                         static_cast<char*>(y) + 32 * n * ybytes, (int)y_bf16);
      return hipGetLastError();
    }
    auto k1 = pre ? linear_skinny<1, GS, (GS > 0)> : linear_skinny<1, GS>;
    const unsigned t1 = (unsigned)(pre ? sk_waves<1, GS, (GS > 0)>() : sk_waves<1, GS, false>()) * kWave;
    auto kernel = m <= 16 ? k1 : (m <= 32 ? k2 : linear_skinny<4, GS, (GS > 0)>);
    const unsigned th = m <= 16 ? t1 : (m <= 32 ? t2 : (unsigned)sk_waves<4, GS, (GS > 0)>() * kWave);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(th), 0, stream, x, packed,
                       sign, scale, scale16, bias, (int)m, (int)n, (int)k, lv, y, (int)y_bf16);
  } else {
    const int64_t tiles_m = (m + kTM - 1) / kTM, tiles_n = (n + kTN - 1) / kTN;
    int sps = 0;
    const int split = GS == 0 ? tiled_split(m, n, k, &sps) : 1;
    if (split > 1) {
      hipLaunchKernelGGL((linear_tiled<false, GS, (GS == 0)>), dim3((unsigned)(tiles_m * tiles_n * split)),
                         dim3(kTThreads), 0, stream, x, packed, sign, scale, scale16, bias, (int)m,
                         (int)n, (int)k, (int)tiles_m, lv, y, (int)y_bf16, sps, part);
      const int64_t count = m * n;
      const int64_t rb = std::min<int64_t>((count + 255) / 256, 8192);
      hipLaunchKernelGGL(linear_split_reduce, dim3((unsigned)rb), dim3(256), 0, stream, part, split,
                         count, (int)n, bias, y, (int)y_bf16);
      return hipGetLastError();
    }
    auto kernel = (k % kTK) ? linear_tiled<true, GS> : linear_tiled<false, GS>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kTThreads), 0, stream, x,
                       packed, sign, scale, scale16, bias, (int)m, (int)n, (int)k, (int)tiles_m,
                       lv, y, (int)y_bf16, 0, nullptr);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                         const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                         const Levels& lv, void* y, bool y_bf16, void* workspace,
                         hipStream_t stream) {
  return launch_linear_any<0>(x, packed, sign, scale, nullptr, bias, m, n, k, lv, y, y_bf16,
                              static_cast<float*>(workspace), stream);
}

// The split-k partial sums of the tiled layer (per-row scales): S planes of
// m x n float32; none for every other path, mid-size m run as slices of x
// rows through the skinny kernel included.
size_t linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= kSkinnyMaxM || mid_m_as_slices(m, n, k, true)) return 0;
  const int split = tiled_split(m, n, k, nullptr);
  if (split <= 1) return 0;
  return ((size_t)split * (size_t)m * (size_t)n * 4u + 255u) & ~size_t(255);
}

hipError_t launch_linear_dense(const uint16_t* x, const uint16_t* wd, const float* bias, int64_t m,
                              int64_t n, int64_t k, void* y, bool y_bf16, hipStream_t stream) {
  // mid-size m as 64-row slices when cheaper, as for the on-chip decoder (the
  // same cost model holds: W' streams at a similar rate, mostly from the
  // Infinity Cache after the first slice)
  if (mid_m_as_slices(m, n, k)) {
    const int64_t ybytes = y_bf16 ? 2 : 4;
    for (int64_t r = 0; r < m; r += kSkinnyMaxM) {
      const int64_t mm = m - r < kSkinnyMaxM ? m - r : kSkinnyMaxM;
      const hipError_t e = launch_linear_dense(x + r * k, wd, bias, mm, n, k,
                                               static_cast<char*>(y) + r * n * ybytes, y_bf16, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (m <= kSkinnyMaxM) {
    const int64_t blocks = (n + kSkRows - 1) / kSkRows;
    auto kernel = m <= 16 ? linear_dense_skinny<1> : (m <= 32 ? linear_dense_skinny<2> : linear_dense_skinny<4>);
    const unsigned th = (m <= 32 ? 16 : 8) * kWave;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(th), 0, stream, x, wd, bias, (int)m, (int)n,
                       (int)k, y, (int)y_bf16);
  } else {
    const int64_t tiles_m = (m + kTM - 1) / kTM, tiles_n = (n + kTN - 1) / kTN;
    auto kernel = (k % kTK) ? linear_dense_tiled<true> : linear_dense_tiled<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kTThreads), 0, stream, x, wd,
                       bias, (int)m, (int)n, (int)k, (int)tiles_m, y, (int)y_bf16);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
//
// Device memory for callers that cannot allocate (code under graph capture,
// serving loops, harnesses that forbid hipMalloc): opq_linear_bits_noalloc
// writes its bfloat16 W' here instead of into a caller workspace.  Every GPU
// the library runs on holds one copy, of kNoAllocScratchBytes, until the
// process ends; calls on one GPU share it, so calls that may overlap there
// race.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels get the address hipGetSymbolAddress reports for the current
// device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

hipError_t launch_linear_grouped(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                                 const uint16_t* scale16, const float* bias, int64_t m, int64_t n,
                                 int64_t k, int gs, const Levels& lv, void* y, bool y_bf16,
                                 void*, hipStream_t stream) {
#define OPQ_GROUP_CASE(G)                                                                       \
  case G:                                                                                       \
    return launch_linear_any<G>(x, packed, sign, nullptr, scale16, bias, m, n, k, lv, y, y_bf16, \
                                nullptr, stream);
  switch (gs) {
    OPQ_GROUP_CASE(32)
    OPQ_GROUP_CASE(64)
    OPQ_GROUP_CASE(128)
    OPQ_GROUP_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef OPQ_GROUP_CASE
}

}  // namespace opq
