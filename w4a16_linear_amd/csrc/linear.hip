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
#include "decode.hpp"
#include "device_common.hpp"
#include "group.hpp"

namespace opq {
namespace {

// ---------------------------------------------------------------- operand order

// x chunk (8 bf16, natural k order) -> the dequantizer's pair order.
__device__ __forceinline__ uint4 sigma_order(uint4 v) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (k0, k2)
  r.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (k4, k6)
  r.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (k1, k3)
  r.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (k5, k7)
  return r;
}

// Output element (row i of a 16-row weight fragment, column c of a 16-column x
// fragment) of v_mfma_f32_16x16x32_bf16 sits in lane 16 * (i / 4) + c,
// register i % 4.
__device__ __forceinline__ void store_y(void* y, bool y_bf16, int64_t at, float v) {
  if (y_bf16) static_cast<uint16_t*>(y)[at] = (uint16_t)bf16_rne(v);
  else static_cast<float*>(y)[at] = v;
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

  const int nbatch = (mine + CH - 1) / CH;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (nbatch > d) load_batch(d, d);

  // Byte planes of the block's 16 row tables: wave w < 4 makes entries
  // 4w .. 4w+3 of row `lane` (a wave-uniform code, so the levels stay in
  // scalar registers).
  if constexpr (GS > 0 && !kPre) build_mant_table(lv, s_mt);
  if (kPre && tid < kSkRows * ngroups) {
    // thread t: the table of group t / 16 of row n0 + t % 16 (all sixteen
    // entries, each with a compile-time level index)
    const float m16 = f16_value(scale16[(int64_t)min(n0 + (tid & (kSkRows - 1)), n - 1) * ngroups +
                                        tid / kSkRows]);
    const RowLut t = make_row_lut(lv, m16);
    *reinterpret_cast<u32x4_t*>(&s_glut[8 * tid]) = u32x4_t{t.lo[0], t.lo[1], t.lo[2], t.lo[3]};
    *reinterpret_cast<u32x4_t*>(&s_glut[8 * tid + 4]) = u32x4_t{t.hi[0], t.hi[1], t.hi[2], t.hi[3]};
  }
  if (GS == 0 && wave < 4 && lane < kSkRows) {
    const float mr = scale[min(n0 + lane, n - 1)];
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
          decode_word_ordered<false>(words[t], sb >> (8 * t), lut, o);
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
// rows [32w, 32w + 32) of the tile (one B fragment) and all 256 x rows: 8
// accumulators of 32x32 (128 fp32 per lane).
//
// Each weight row is decoded once per tile step, in registers: a lane
// dequantizes one packed word (the eight k values it supplies to the B
// operand) with its row's table held as byte planes (v_perm lookups).  Lanes
// 0..31 take words 0..3 of the 8-word k step and lanes 32..63 words 4..7, so
// sub-step s contracts k-blocks {s, 4 + s}; the x fragments read from LDS use
// the same k-blocks.  Within a k-block the dequantizer emits bf16 pairs in the
// order (k0,k2) (k4,k6) (k1,k3) (k5,k7); x is stored to LDS in that order too
// (two stages, rows XOR-swizzled by 16-byte chunk).

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kAStage = kTM * kTK;                 // bf16 per stage

// LDS element offset of 16-byte chunk c of tile row r.  A row is 128 bytes
// (32 banks), so rows alternate bank halves; XOR-ing the chunk with bits 1..3
// of the row spreads any 16 consecutive rows over all 64 banks, which keeps the
// 16-lane passes of ds_read_b128 conflict-free.
__device__ __forceinline__ int a_off(int r, int c) { return r * kTK + ((c ^ ((r >> 1) & 7)) << 3); }

// The weights are staged through LDS.  Every two k steps the block loads its
// 256 weight rows x 64 bytes of codes (and the two steps' sign words) with
// loads in which each group of four lanes reads 64 contiguous bytes, two steps
// before use, into one of two LDS stages of 80-byte row records (codes of the
// two steps, then their sign words: a stride that keeps the 32-row fragment
// reads below free of bank conflicts).  Wave w reads the codes of its rows
// 32w .. 32w + 31 for a step with one ds_read_b128 and one ds_read_b32 per
// lane.  (Loading the B-operand layout straight from HBM made every dwordx4
// touch 32 rows.)
constexpr int kWRec = 20;  // uint32 per weight row record: 16 code words + 4 sign words

//
// GS > 0: the group-wise form (group.hpp).  The lane's table is rebuilt from
// the LDS significand table before the first sub-step of every k step; the
// float16 group maxima are loaded two steps ahead.
template <bool kHalfTail, int GS>
__global__ __launch_bounds__(512, 1) void linear_mfma_ws(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint32_t* __restrict__ sign, const float* __restrict__ scale,
    const uint16_t* __restrict__ scale16, const float* __restrict__ bias, int m, int n, int k,
    int tiles_m, Levels lv, void* __restrict__ y, int y_bf16) {
  constexpr int kThreads = 512;
  constexpr int XCH = kTM * kTK / 8 / kThreads;     // x chunks each thread stages per step (4)
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2 * kAStage];
  __shared__ __attribute__((aligned(16))) uint32_t s_w[2][kTN][kWRec];
  __shared__ __attribute__((aligned(16))) uint32_t s_mt[GS ? kMantissas * 8 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int m0 = tile_m * kTM;
  const int n0 = tile_n * kTN;
  const int nw = n0 + wave * 32;                  // first weight row of this wave
  const int g = lane >> 5;                        // which half of the k step
  const int kwords = k / 8, swords = k / 32;
  const int nsteps = (k + kTK - 1) / kTK;
  const int npairs = (nsteps + 1) / 2;

  const int brow = nw + (lane & 31);
  RowLut lut;
  if constexpr (GS == 0) lut = make_row_lut(lv, scale[min(brow, n - 1)]);
  // GS > 0: float16 max of this lane's group in step kt (its half of the step)
  const int ngroups = GS ? k / GS : 1;
  const uint16_t* hrow = GS ? scale16 + (int64_t)min(brow, n - 1) * ngroups : nullptr;
  auto load_h = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    if constexpr (GS > 0)
      return hrow[min((min(kt, nsteps - 1) * kTK + 32 * g) / GS, ngroups - 1)];
    else
      return 0u;
  };
  uint32_t h_next = 0u, h_load = 0u;  // maxima of steps kt + 1 and kt + 2

  // Weight loads for step pair p (steps 2p, 2p + 1): thread t moves 16 code
  // bytes (quarter t % 4) of tile rows t/4 and t/4 + 128, and sign words
  // 2(t%2), 2(t%2) + 1 of the pair for tile row t/2.  Rows past n read row
  // n - 1; parts past k read the row's last 16 code bytes or last sign word
  // (only ever met by zeroed fragments or steps that are never used).
  const int wq = tid & 3;
  const int n0c = min(n0, n - 1);
  const char* pbase = reinterpret_cast<const char*>(packed + (int64_t)n0c * kwords);
  const uint32_t* sbase = sign + (int64_t)n0c * swords;
  const uint32_t pa_off = (uint32_t)(min(n0 + (tid >> 2), n - 1) - n0c) * (uint32_t)kwords * 4u;
  const uint32_t pb_off = (uint32_t)(min(n0 + 128 + (tid >> 2), n - 1) - n0c) * (uint32_t)kwords * 4u;
  const uint32_t s_off = (uint32_t)(min(n0 + (tid >> 1), n - 1) - n0c) * (uint32_t)swords;
  uint4 wv[2];
  uint32_t wsg[2];
  auto load_w = [&](int p) __attribute__((always_inline)) {
    const int pc = min(p, npairs - 1);
    const uint32_t e = (uint32_t)min(pc * 2 * kTK + 32 * wq, k - 32);  // first element of the part
    wv[0] = *reinterpret_cast<const uint4*>(pbase + pa_off + e / 2u);
    wv[1] = *reinterpret_cast<const uint4*>(pbase + pb_off + e / 2u);
#pragma unroll
    for (int i = 0; i < 2; ++i) wsg[i] = sbase[s_off + (uint32_t)min(pc * 4 + 2 * (tid & 1) + i, swords - 1)];
  };
  auto store_w = [&](int p) __attribute__((always_inline)) {
    uint32_t (*st)[kWRec] = s_w[p & 1];
    *reinterpret_cast<u32x4_t*>(&st[tid >> 2][4 * wq]) = u32x4_t{wv[0].x, wv[0].y, wv[0].z, wv[0].w};
    *reinterpret_cast<u32x4_t*>(&st[128 + (tid >> 2)][4 * wq]) = u32x4_t{wv[1].x, wv[1].y, wv[1].z, wv[1].w};
#pragma unroll
    for (int i = 0; i < 2; ++i) st[tid >> 1][16 + 2 * (tid & 1) + i] = wsg[i];
  };
  // This lane's codes and sign word of step kt (from stage (kt/2) & 1).
  auto read_w = [&](int kt, uint4& pw, uint32_t& sw) __attribute__((always_inline)) {
    const uint32_t* rec = s_w[(kt >> 1) & 1][wave * 32 + (lane & 31)];
    const int half = kt & 1;
    pw = *reinterpret_cast<const uint4*>(rec + 8 * half + 4 * g);
    sw = rec[16 + 2 * half + g];
  };

  const char* xbase = reinterpret_cast<const char*>(x + (int64_t)m0 * k);
  uint32_t x_off[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + kThreads * i;
    const int r = min(m0 + (c >> 3), m - 1) - m0;
    x_off[i] = ((uint32_t)r * (uint32_t)k + 8u * (uint32_t)(c & 7)) * 2u;
  }
  auto load_a = [&](int kt, uint4 (&xa)[XCH]) __attribute__((always_inline)) {
    const int kc = min(kt, nsteps - 1) * kTK;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      uint32_t off = x_off[i] + (uint32_t)kc * 2u;
      if constexpr (kHalfTail) {
        const int c = tid + kThreads * i;
        if (kc + 8 * (c & 7) >= k) off -= 64u;  // step back into the row
      }
      xa[i] = *reinterpret_cast<const uint4*>(xbase + off);
    }
  };
  auto store_a = [&](int stage, const uint4 (&xa)[XCH]) __attribute__((always_inline)) {
    uint16_t* base = s_a + stage * kAStage;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + kThreads * i;
      const uint4 v = sigma_order(xa[i]);
      *reinterpret_cast<u32x4_t*>(base + a_off(c >> 3, c & 7)) = u32x4_t{v.x, v.y, v.z, v.w};
    }
  };

  floatx16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

  auto dequant_b = [&](int kt, int s, const uint4& pwv, uint32_t swv, bf16x8_t& b)
      __attribute__((always_inline)) {
    const uint32_t words[4] = {pwv.x, pwv.y, pwv.z, pwv.w};
    uint32_t o[4];
    dequant_word(words[s], swv >> (8 * s), lut, o);
    if constexpr (kHalfTail) {
      if (kt == nsteps - 1 && g == 1) o[0] = o[1] = o[2] = o[3] = 0u;
    }
    b = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  };
  auto read_a = [&](const uint16_t* sa, int s, bf16x8_t (&a)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
      a[mi] = *reinterpret_cast<const bf16x8_t*>(sa + a_off(mi * 32 + (lane & 31), 4 * g + s));
  };

  // Step pair q is stored at step 2q - 2 (sub-step 0) from registers loaded at
  // step 2q - 4, and first read at step 2q - 1 after that step's barrier; the
  // stage it overwrites last served step 2q - 3, read at step 2q - 4.
  uint4 pw;        // codes of the current step (read at the previous step's sub-step 3)
  uint32_t sw;
  uint4 xa[XCH];
  bf16x8_t a_frag[8], b_buf[2];  // one x fragment set: its registers keep the kernel clear of scratch
  if (nsteps > 0) {
    uint32_t h0 = 0u;
    if constexpr (GS > 0) {
      h0 = load_h(0);
      h_next = load_h(1);
    }
    load_a(0, xa);
    load_w(0);
    if constexpr (GS > 0) build_mant_table(lv, s_mt);
    store_a(0, xa);
    store_w(0);
    load_a(1, xa);
    load_w(1);
    __syncthreads();
    if constexpr (GS > 0) lut = group_lut(s_mt, h0);
    read_w(0, pw, sw);
    read_a(s_a, 0, a_frag);
    dequant_b(0, 0, pw, sw, b_buf[0]);
  }

  auto step = [&](int kt, bool even) __attribute__((always_inline)) {
    const int stage = kt & 1;
    const uint16_t* sa = s_a + stage * kAStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      // The next sub-step's x fragments are read once this one's MFMAs are
      // issued; the other wave on the SIMD covers the LDS latency.
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag[mi], b_buf[cur], acc[mi], 0, 0, 0);
      if (s < 3) {
        read_a(sa, s + 1, a_frag);
        dequant_b(kt, s + 1, pw, sw, b_buf[nxt]);
      } else {
        __syncthreads();
        read_a(s_a + (stage ^ 1) * kAStage, 0, a_frag);
        read_w(kt + 1, pw, sw);  // this step's words are dead after sub-step 2
        if constexpr (GS > 0) {
          // the table of step kt + 1, when it starts a new group (every step
          // for groups of 32 and 64: the two halves of a step differ or the
          // group is one step long)
          if (GS <= kTK || ((kt + 1) * kTK) % GS == 0) lut = group_lut(s_mt, h_next);
          h_next = h_load;
        }
        dequant_b(kt + 1, 0, pw, sw, b_buf[nxt]);
      }
      if (s == 0) {
        if constexpr (GS > 0) h_load = load_h(kt + 2);
        store_a(stage ^ 1, xa);
        load_a(kt + 2, xa);
        if (even) {
          store_w(kt / 2 + 1);
          load_w(kt / 2 + 2);
        }
      }
    }
  };
  int kt = 0;
  for (; kt + 1 < nsteps; kt += 2) {
    step(kt, true);
    step(kt + 1, false);
  }
  if (kt < nsteps) step(kt, true);

  // 32x32 accumulator layout: register e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
  const float bv = (bias && brow < n) ? bias[brow] : 0.0f;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
      if (row < m && brow < n) store_y(y, y_bf16, (int64_t)row * n + brow, acc[mi][e] + bv);
    }
}

}  // namespace

size_t linear_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

namespace {

template <int GS>
hipError_t launch_linear_any(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                             const float* scale, const uint16_t* scale16, const float* bias,
                             int64_t m, int64_t n, int64_t k, const Levels& lv, void* y,
                             bool y_bf16, hipStream_t stream) {
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
    auto kernel = (k % kTK) ? linear_mfma_ws<true, GS> : linear_mfma_ws<false, GS>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream, x,
                       packed, sign, scale, scale16, bias, (int)m, (int)n, (int)k, (int)tiles_m,
                       lv, y, (int)y_bf16);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                         const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                         const Levels& lv, void* y, bool y_bf16, void*, hipStream_t stream) {
  return launch_linear_any<0>(x, packed, sign, scale, nullptr, bias, m, n, k, lv, y, y_bf16,
                              stream);
}

hipError_t launch_linear_grouped(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                                 const uint16_t* scale16, const float* bias, int64_t m, int64_t n,
                                 int64_t k, int gs, const Levels& lv, void* y, bool y_bf16,
                                 void*, hipStream_t stream) {
#define OPQ_GROUP_CASE(G)                                                                       \
  case G:                                                                                       \
    return launch_linear_any<G>(x, packed, sign, nullptr, scale16, bias, m, n, k, lv, y, y_bf16, \
                                stream);
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
