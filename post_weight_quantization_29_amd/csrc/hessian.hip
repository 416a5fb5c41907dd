// Calibration Hessian H += 2 X^T X (GPTQ practice page m.lqnn.cn/news/117696,
// section 2.1: the Hessian comes from the layer's input activations).
//
// X is token-major [n_tokens x d], so both MFMA operands have the token index
// as their contraction index and channels contiguous in memory.  Tiles of X
// are copied to LDS exactly as laid out in HBM (channel-contiguous rows) and
// the K-contiguous MFMA operands are produced by the gfx950 transposing LDS
// read ds_read_b64_tr_b16.  Only lower-triangle tiles are computed; the token
// range is split so that enough workgroups exist, each split writes its
// partial tile in the MFMA register order, and a second kernel adds the
// partials in a fixed order into H and mirrors off-diagonal tiles.
#include "common.h"
#include "split3.h"

#include <mutex>

namespace gptq {

// ---------------------------------------------------------------------------
// tile bookkeeping
// ---------------------------------------------------------------------------
GPTQ_DEV void tri_tile(int q, int& I, int& J) {
  // q enumerates (I, J), I >= J, row by row: q = I(I+1)/2 + J
  int i = (int)((sqrtf(8.0f * (float)q + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= q) ++i;
  while (i * (i + 1) / 2 > q) --i;
  I = i;
  J = q - i * (i + 1) / 2;
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD = w % 8), each
// with its own L2.  Tiles are ordered by 4x4 super-blocks of the lower
// triangle and cut into 8 contiguous chunks, one per XCD, so the tiles an XCD
// runs share few channel panels; inside an XCD the items run split-major, so
// the co-resident workgroups read the same token range.  Returns false for the
// padding workgroups past the last tile of a chunk.
constexpr int kXCD = 8;
constexpr int kSB = 4;

GPTQ_DEV bool xcd_item(int w, int nt, int ntiles, int splits, int& s, int& I, int& J) {
  const int chunk = (ntiles + kXCD - 1) / kXCD;
  const int x = w % kXCD, k = w / kXCD;
  s = k / chunk;
  const int L = x * chunk + (k - s * chunk);
  if (s >= splits || L >= ntiles) return false;
  // walk the super-blocks (row-major over the lower triangle) to tile number L
  const int nsb = (nt + kSB - 1) / kSB;
  int rem = L;
  for (int ib = 0; ib < nsb; ++ib) {
    const int h = min(kSB, nt - ib * kSB);
    for (int jb = 0; jb <= ib; ++jb) {
      const int wdt = min(kSB, nt - jb * kSB);
      const int cnt = (ib == jb) ? h * (h + 1) / 2 : h * wdt;
      if (rem < cnt) {
        if (ib == jb) {
          int r = 0;
          while (rem >= r + 1) { rem -= r + 1; ++r; }
          I = ib * kSB + r;
          J = jb * kSB + rem;
        } else {
          I = ib * kSB + rem / wdt;
          J = jb * kSB + rem % wdt;
        }
        return true;
      }
      rem -= cnt;
    }
  }
  return false;
}

GPTQ_DEV int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// ---------------------------------------------------------------------------
// 16-bit inputs: bf16 / fp16, v_mfma_f32_32x32x16_{bf16,f16}
// Workgroup tile 256x256, 4 waves (2x2) of 128x128, 32 tokens per stage.
//
// Stages are copied HBM -> LDS by buffer_load ... lds (16 bytes per lane, the
// 64 lanes of one instruction fill 1 KB of LDS in lane order) into a ring of
// five slots (160 KB, all of a CU's LDS): stage kk+3 streams in while stage kk
// is multiplied, so a copy has about three stages to land, with no staging
// registers.  (Four slots, two stages of slack, cost 8 % at 8192 x 28672, where
// the paced workgroups run at 2 GHz and the copies' latency showed.)  The 16 copies a wave issues per stage are interleaved one per
// MFMA with the first k-slice, so the MFMA pipe keeps running while the
// address unit takes them.  A stage row (one token, 256 channels) is 512 bytes, unpadded;
// its 16-byte chunk c sits at slot c ^ 4*(row % 4), which keeps the
// transposing operand reads free of bank conflicts (the DMA side applies the
// swizzle by permuting the lanes' source addresses).  Tokens past the end and
// channels past d read as zero through the buffer descriptor's range.
// ---------------------------------------------------------------------------
constexpr int kT16 = 256;          // tile edge (channels)
constexpr int kK16 = 32;           // tokens per stage (2 k-slices of 16)
constexpr int kSlots16 = 5;        // LDS ring slots
constexpr int kRow16 = kT16;       // LDS row pitch in elements (512 bytes)
constexpr int kStage16 = kK16 * kRow16;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds: each lane's 16 bytes go to LDS at M0 + 16*lane.
// Issued from asm so that the compiler does not model an outstanding LDS write
// (it would otherwise drain every copy in flight before each LDS read); the
// kernel waits for the copies itself with counted s_waitcnt vmcnt.  All
// operands are wave-uniform except the per-lane offset.
GPTQ_DEV void dma16(i32x4_t rsrc, const void* lds_dst, int voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS const void*)lds_dst);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(rsrc[0]);
  r[1] = __builtin_amdgcn_readfirstlane(rsrc[1]);
  r[2] = __builtin_amdgcn_readfirstlane(rsrc[2]);
  r[3] = __builtin_amdgcn_readfirstlane(rsrc[3]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r)
               : "memory", "m0");
}

// workgroup barrier that also stops the compiler from moving memory accesses
// across it, without the fence's drain of outstanding global loads
GPTQ_DEV void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename T> struct Op16;
template <> struct Op16<__bf16> {
  typedef bf16x8_t v8;
  typedef bf16x4_t v4;
  static GPTQ_DEV v4 tr(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4*)(uintptr_t)addr);
  }
  static GPTQ_DEV f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static GPTQ_DEV float to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
};
template <> struct Op16<_Float16> {
  typedef f16x8_t v8;
  typedef f16x4_t v4;
  typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  static GPTQ_DEV v4 tr(uint32_t addr) {
    raw4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS raw4*)(uintptr_t)addr);
    return __builtin_bit_cast(v4, r);
  }
  static GPTQ_DEV f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static GPTQ_DEV float to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
};

// element offset of (token row, channel) inside a stage
GPTQ_DEV int swz16(int row, int ch) { return row * kRow16 + ((((ch >> 3) ^ (4 * (row & 3)))) << 3) + (ch & 7); }

// Transposing read at an LDS byte address (the constant part of the address
// folds into the instruction's offset field).
template <typename T>
GPTQ_DEV typename Op16<T>::v4 tr_at(uint32_t addr) {
  return Op16<T>::tr(addr);
}

// Per-lane byte offset, inside a stage, of the first of a lane's two
// transposing reads for the 32-channel block starting at cbase, k-slice 0.
// The read gives lane j of each 16-lane group g the element (4e + (j%16)/4,
// j%4) of the group's 16x4 block of 64-bit loads; pointing lane 16g+4a+b at
// token 8*(g/2) + a (+4 for the second read) and channels cbase + 16*(g%2) +
// 4b .. +3 hands lane l channel cbase + l%32 at tokens 8*(l/32) + 0..7, i.e.
// MFMA k-slot order.  Token rows of one read differ by multiples of 4, so the
// swizzle term 4*(row%4) = 4a is fixed per lane and k-slice s / second read
// only add 16*s*512 and 4*512 bytes.
GPTQ_DEV uint32_t lane_op_offset(int cbase, int lane) {
  const int g = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
  const int tok = 8 * (g >> 1) + a;
  const int ch = cbase + 16 * (g & 1) + 4 * b;
  return 2u * (uint32_t)swz16(tok, ch);
}

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left open)
template <int N>
GPTQ_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
GPTQ_DEV void wait_vm0() { wait_vm<0>(); }

// The fp64 diagonal keys of 16-bit inputs (the desc_act order) are not summed
// here: a separate streaming pass over X does it (see hessian_launch).
//
// Partial layout (floats): [work item][wave 4][block 16 = mb*4+nb][reg 16][lane 64]
// Pacing.  A workgroup streams every token of its tile, so over a tile's
// thousands of stages the co-resident workgroups of an XCD drift apart by
// far more than the few stages of channel panels their L2 can hold for one
// another, and each re-reads the panels it shares from memory (at 8192 x
// 28672, 100x the activations' bytes per call).  Each workgroup therefore
// publishes the stages it has done in its slot of its XCD's 64-slot row
// (pace[x][c]) every kPaceEvery stage groups, and wave 0 then waits while it
// is more than kPaceLag stages ahead of the slowest workgroup of its XCD
// (finished ones publish ~0u).  A poll is rare because its load must be
// waited for with every copy still in flight (the copies are issued by asm
// the compiler cannot count), which drains the stage ring: polling every
// group of five stages cost 14% of the call.  The wait is bounded
// (kPaceSpin polls); a workgroup whose wait runs out stops pacing, so
// residency problems cost time, never a hang.  Only timing depends on it:
// every sum is the same.
constexpr unsigned kPaceLag = 8;
constexpr int kPaceEvery = 16;      // stage groups (of kSlots16 stages) between polls
constexpr int kPaceSpin = 4096;
constexpr int kPaceSlots = 64;

GPTQ_DEV unsigned wave_min_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, o));
  return v;
}

// Update modes: fp32 products on the 16-bit tile loop.  An fp32 operand x is
// scaled by a power of two per output row or column, 2^(14 - e) with e the
// exponent of that row's or column's largest |x| (exact; the largest then
// lies in [2^14, 2^15), inside fp16's range), and split into two fp16 pieces
// h = fp16(x'), l = fp16(x' - h) (the difference is exact in fp32 and
// |x' - h - l| <= 2^-22 |x'|).  A product of two operands is the sum of the
// three piece products lh, hl, hh (the dropped ll and the split residuals
// are <= 3 2^-22 of the product, below what the fp32 accumulation of the
// contraction already carries), so each fp32 product costs three fp16
// products on v_mfma_f32_32x32x16_f16.  The contraction runs over 3K virtual
// tokens, one segment of K per piece product, smallest first, so the
// accumulator grows from the 2^-11-scale products to the hh ones and only
// those are rounded at the scale of the result; the accumulators start from
// zero and C takes C + alpha 2^(eA_i + eB_j - 28) acc once at the end (the
// power of two exact), through buffer resources.
// MODE 1 (symmetric): C[upper] -= P^T P for an fp32 panel P (K x n, planes
// h, l of X, row pitch n); tiles run as upper tiles (I <= J) and the strictly
// lower 128-block of a diagonal tile is left alone.  n is a multiple of 128,
// so a wave's 128 x 128 block is wholly inside C or outside.
// MODE 2 (general): C (m x n) = beta C + alpha A^T B, alpha = +-1, beta 0 or
// 1, for fp32 A (K x m) and B (K x n) given as their planes h, l (A's from X,
// row pitch m = d; B's from B, row pitch n), over every tile of C, stores
// guarded element by element.
// Piece of each of the three segments (nibble g of kSegA / kSegB: 0 = h,
// 1 = l): l h, h l, h h.
constexpr int kSegs = 3;
constexpr int kSegA = 0x001;
constexpr int kSegB = 0x010;

struct Split3Args {
  float* C;         // MODE 1: n x n; MODE 2: m x n; row pitch ldc
  int ldc;
  int kseg;         // K, a multiple of the 32-token stage
  int64_t plane;    // elements from one plane of X to the next (h, l)
  const _Float16* B;  // MODE 2: B's planes h, l (row pitch n)
  int64_t planeB;   // MODE 2: elements from one plane of B to the next
  const unsigned* sA;  // largest |x| (float bits) of each row of C's operand A (MODE 1: of P's columns)
  const unsigned* sB;  // the same for the columns of C (MODE 1: sA again)
  int n;            // MODE 2: columns of C and of B
  int ntn;          // MODE 2: 256-wide tile columns
  int neg;          // MODE 2: alpha = -1 (MODE 1: always)
  int beta;         // MODE 2: 1 = C is read and accumulated into, 0 = C is overwritten
  int kmode;        // MODE 2 contraction of tile (I, J): 0 all K; 1 k >= 256 I; 2 k < min(K, 256 (J + 1))
  unsigned* queue;  // MODE 2, kmode != 0: per-XCD item counters (x * 32), zero at launch
};

// exponent e of a row's or column's largest |x| (given as float bits): its
// pieces are taken of x 2^(14 - e); an all-zero row or column takes e = 0
GPTQ_DEV int piece_exp(unsigned maxbits) {
  const float m = __builtin_bit_cast(float, maxbits);
  return (m > 0.0f) ? ilogbf(m) : 0;
}

// MODE 2 tile order: strips of kSB tile rows cut into column-blocks (the kSB
// tiles of one tile column of a strip), dealt round-robin to the 8 XCDs:
// item k of XCD x is tile k % kSB of column-block (k / kSB) * 8 + x, so a
// round of an XCD's 32 co-resident workgroups shares 4 A panels and 8 B
// panels, and with triangular operands (the tile's contraction grows with
// its row or column) every XCD gets the same mix of long and short tiles.
// Items past C's last tile row return false.
GPTQ_DEV bool rect_item(int x, int k, int mt, int ntn, int& I, int& J) {
  const int q = (k / kSB) * kXCD + x;
  const int sb = q / ntn;
  I = sb * kSB + k % kSB;
  J = q - sb * ntn;
  return I < mt;
}

// items per XCD of the MODE 2 order
GPTQ_DEV int rect_items_per_xcd(int mt, int ntn) {
  const int nsb = (mt + kSB - 1) / kSB;
  return ((nsb * ntn + kXCD - 1) / kXCD) * kSB;
}

template <typename T, bool PACE, int MODE>
__global__ __launch_bounds__(256, 1) void syrk16_kernel(const T* __restrict__ X, int64_t n_tokens,
                                                         int d, int nt, int ntiles, int splits,
                                                         int nk, float* __restrict__ partial,
                                                         unsigned* __restrict__ pace, Split3Args up) {
  constexpr bool UPD = MODE != 0;
  static_assert(!(UPD && PACE), "the update modes read cached planes: no pacing");
  static_assert(MODE != 2 || sizeof(T) == 2, "planes are 16-bit");
  __shared__ __attribute__((aligned(16))) T sA[kSlots16][kStage16];
  __shared__ __attribute__((aligned(16))) T sB[kSlots16][kStage16];
  constexpr uint32_t kSlotBytes = kStage16 * 2;    // 16 KB
  constexpr uint32_t kSliceBytes = 16 * kRow16 * 2; // 16 token rows
  constexpr int NI = kK16 / 8;                     // copies per panel per lane per stage
  constexpr int NKS = kK16 / 16;                   // k-slices per stage

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const uint32_t rowB_bytes = (MODE == 2) ? (uint32_t)up.n * 2u : row_bytes;   // B's row pitch
  const int dB = (MODE == 2) ? up.n : d;                                     // B's channels
  const uint32_t ldsA = (uint32_t)(uintptr_t)(LDS_AS const void*)&sA[0][0];
  const uint32_t ldsB = (uint32_t)(uintptr_t)(LDS_AS const void*)&sB[0][0];

  uint32_t offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    offA[i] = lane_op_offset(wm * 128 + i * 32, lane);
    offB[i] = lane_op_offset(wn * 128 + i * 32, lane);
  }

  // Persistent: workgroup (x = XCD, c) runs items c, c + nper, c + 2*nper, ... of
  // XCD x's list, so the workgroups of an XCD move through the list in rounds
  // and those sharing channel panels read the same tokens at the same time.
  const int x = blockIdx.x % kXCD, c = blockIdx.x / kXCD, nper = gridDim.x / kXCD;
  // MODE 2 with triangular bounds: the items of an XCD's list are taken one
  // by one from the XCD's counter, longest contraction first (its strips run
  // along the dimension the contraction length depends on), so its
  // workgroups stay evenly loaded whatever the lengths (a fixed deal of
  // items to workgroups left the busiest with 1.1-1.4x the mean)
  const bool dyn = (MODE == 2) && up.queue != nullptr;
  const bool tcol = (MODE == 2) && up.kmode == 2;   // strips of tile columns
  const int per_xcd = (MODE == 2) ? (tcol ? rect_items_per_xcd(up.ntn, nt) : rect_items_per_xcd(nt, up.ntn))
                                  : ((ntiles + kXCD - 1) / kXCD) * splits;
  unsigned* prow = PACE ? pace + x * kPaceSlots : nullptr;
  bool pacing = PACE && (wave == 0) && (nper <= kPaceSlots);
  unsigned done = 0;                             // stages done (skipped items included)
  // wave 0: publish `progress`, then wait (bounded) while more than kPaceLag
  // stages ahead of the XCD's slowest workgroup
  auto pace_at = [&](unsigned progress) {
    if (!PACE || !pacing) return;
    if (lane == 0) __hip_atomic_store(prow + c, progress, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0;; ++it) {
      const unsigned v = (lane < nper) ? __hip_atomic_load(prow + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                       : ~0u;
      if (wave_min_u32(v) + kPaceLag >= progress) break;
      if (it == kPaceSpin) {
        // stop pacing, and let no one wait on this workgroup any more
        pacing = false;
        if (lane == 0) __hip_atomic_store(prow + c, ~0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  for (int kidx = c;; kidx += nper) {
  if (dyn) {
    // every wave is done with the ring (and the previous item's exponent
    // tables); thread 0 takes the next item and hands it over through LDS
    wait_vm0();
    lds_barrier();
    unsigned* slot = reinterpret_cast<unsigned*>(&sA[0][0]);
    if (tid == 0) *slot = atomicAdd(up.queue + x * 32, 1u);
    __syncthreads();
    kidx = __builtin_amdgcn_readfirstlane((int)*slot);
  }
  if (kidx >= per_xcd) break;
  int s = 0, I, J;
  if (MODE == 2 ? !(tcol ? rect_item(x, kidx, up.ntn, nt, J, I) : rect_item(x, kidx, nt, up.ntn, I, J))
                : !xcd_item(kidx * kXCD + x, nt, ntiles, splits, s, I, J)) {
    // a padding item: count its stages as done so the others do not wait on it
    const int sp = kidx / ((ntiles + kXCD - 1) / kXCD);
    if (PACE && sp < splits) done += (unsigned)((int64_t)nk * (sp + 1) / splits - (int64_t)nk * sp / splits);
    continue;
  }
  s = __builtin_amdgcn_readfirstlane(s);
  I = __builtin_amdgcn_readfirstlane(I);
  J = __builtin_amdgcn_readfirstlane(J);
  const int w = s * ntiles + tri_index(I, J);     // partial slot
  if (MODE == 2 && up.kmode == 2) J = up.ntn - 1 - J;   // longest contractions first
  if (MODE == 1) {
    const int t = I;
    I = J;
    J = t;
  }
  // MODE 2: the tile's contraction [klo, khi) (triangular operands), 6 segments of pseg stages
  int klo = 0, pseg = 0;
  if constexpr (MODE == 2) {
    int khi = up.kseg;
    if (up.kmode == 1) klo = I * kT16;
    if (up.kmode == 2) khi = min(up.kseg, (J + 1) * kT16);
    pseg = __builtin_amdgcn_readfirstlane((khi - klo) / kK16);
    klo = __builtin_amdgcn_readfirstlane(klo);
  }
  const int ks0 = (MODE == 2) ? 0 : __builtin_amdgcn_readfirstlane((int)((int64_t)nk * s / splits));
  const int ks1 = (MODE == 2) ? kSegs * pseg : __builtin_amdgcn_readfirstlane((int)((int64_t)nk * (s + 1) / splits));

  // copies of the previous item (and its stores) are complete and every wave
  // is done with its LDS
  wait_vm0();
  lds_barrier();

  // DMA assignment: copy i of wave v fills stage rows R = 8i+2v (lanes 0-31)
  // and 8i+2v+1 (lanes 32-63); lane slot L%32 of row R takes chunk
  // (L%32) ^ 4(R%4), i.e. channels 8*that .. +7 of the panel.  R%4 does not
  // depend on i.
  int voffA[NI], voffB[NI];
  {
    const int R = 2 * wave + (lane >> 5);
    const int cc = (lane & 31) ^ (4 * (R & 3));
    const int chA = I * kT16 + 8 * cc, chB = J * kT16 + 8 * cc;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      voffA[i] = (chA < d) ? (int)((uint32_t)(R + 8 * i) * row_bytes + chA * 2) : 0x7ffffff0;
      voffB[i] = (chB < dB) ? (int)((uint32_t)(R + 8 * i) * rowB_bytes + chB * 2) : 0x7ffffff0;
    }
  }
  // buffer descriptor of stage kk (rows past the end, or kk outside this
  // split, read as zero)
  auto make_rsrc = [&](uint64_t base, int64_t rows, uint32_t rb) {
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)(rows * rb));
    r[3] = 0x00020000;
    return r;
  };
  // A and B descriptors of stage kk (the same except in the update mode)
  // update modes: stage kk is stage seg_i of segment seg_g; the calls below
  // come in stage order from ks0 = 0, so the pair is advanced instead of
  // divided out of kk
  const int seg_len = (MODE == 1) ? up.kseg / kK16 : pseg;
  int seg_g = 0, seg_i = 0;
  auto stage_rsrc = [&](int kk, i32x4_t& rA, i32x4_t& rB) {
    const int64_t t0 = (int64_t)kk * kK16;
    const int64_t rows = (kk < ks1) ? min<int64_t>(kK16, n_tokens - t0) : 0;
    int g = 0;
    int64_t row = 0;
    if constexpr (UPD) {
      g = min(seg_g, kSegs - 1);         // stages past the tile's last one read nothing (rows = 0)
      row = klo + (int64_t)seg_i * kK16;
      if (++seg_i == seg_len) {
        seg_i = 0;
        ++seg_g;
      }
    }
    if constexpr (MODE == 1) {
      // segment g = 0..2 reads pieces (l,h) (h,l) (h,h) of (P, P)
      const int pa = (kSegA >> (4 * g)) & 0xF, pb = (kSegB >> (4 * g)) & 0xF;
      rA = make_rsrc(reinterpret_cast<uint64_t>(X + pa * up.plane) + (uint64_t)row * row_bytes, rows, row_bytes);
      rB = make_rsrc(reinterpret_cast<uint64_t>(X + pb * up.plane) + (uint64_t)row * row_bytes, rows, row_bytes);
    } else if constexpr (MODE == 2) {
      // segment g = 0..2 reads pieces (l,h) (h,l) (h,h) of (A, B)
      const int pa = (kSegA >> (4 * g)) & 0xF, pb = (kSegB >> (4 * g)) & 0xF;
      rA = make_rsrc(reinterpret_cast<uint64_t>(X + pa * up.plane) + (uint64_t)row * row_bytes, rows, row_bytes);
      rB = make_rsrc(reinterpret_cast<uint64_t>(up.B + pb * up.planeB) + (uint64_t)row * rowB_bytes, rows,
                     rowB_bytes);
    } else {
      rA = make_rsrc(reinterpret_cast<uint64_t>(X) + (uint64_t)t0 * row_bytes, rows, row_bytes);
      rB = rA;
    }
  };
  // copy n (0..2*NI-1) of stage kk's DMA into slot `slot`
  auto dma = [&](const i32x4_t& rA, const i32x4_t& rB, int slot, int n) {
    const i32x4_t& r = (n < NI) ? rA : rB;
    const int i = n % NI;
    const uint32_t dst = ((n < NI) ? ldsA : ldsB) + (uint32_t)slot * kSlotBytes + 4096u * i + 1024u * wave;
    const int voff = (n < NI) ? voffA[i] : voffB[i];
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(r)
                 : "memory", "m0");
  };


  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // update modes: this wave's 128 x 128 block of C (rows from tile I,
  // columns from tile J).  The accumulators start from zero and C is read
  // and added once after the contraction (as in the fp32 tiles): the 6K
  // additions are then rounded at the scale of the update, not of C.
  const int cm0 = I * kT16 + wm * 128, cn0 = J * kT16 + wn * 128;
  const bool cwrite = (MODE == 1) ? (!(I == J && wm == 1 && wn == 0) && cm0 < d && cn0 < d)
                                  : (MODE == 2 && cm0 < d && cn0 < dB);
  // MODE 2: element (i, j, r) of the block is row cm0 + crow(i, r), column
  // cn0 + j*32 + lane%32
  auto c_in = [&](int i, int j, int r) {
    return cm0 + 4 * (lane >> 5) + i * 32 + 8 * (r >> 2) + (r & 3) < d && cn0 + (lane & 31) + j * 32 < dB;
  };

  if (ks0 < ks1) {
    // Ring of kSlots16 stage slots.  The sync point of stage k sits before
    // the last k-slice of stage k-1: there every wave has waited for its own
    // copies of stage k (so after the barrier stage k is complete for all) and
    // has finished the earlier slices of stage k-1 (so stage k-2's slot is
    // free and receives stage k + kSlots16 - 2).  The last slice of a stage
    // then overlaps its MFMAs with the reads of the next stage's first slice
    // and with the next copies, issued one every second MFMA (in a burst
    // they filled the address unit's queue and held the MFMA stream up).
    constexpr int kInFlight = kSlots16 - 3;        // later stages still in flight at a sync point
    static_assert(kSlots16 >= 3 && NKS % 2 == 0 && 2 * NI == 8, "ring layout: 8 copies over a slice's 16 MFMAs");
#pragma unroll
    for (int a = 0; a <= kSlots16 - 3; ++a) {
      i32x4_t r0A, r0B;
      stage_rsrc(ks0 + a, r0A, r0B);
#pragma unroll
      for (int n = 0; n < 2 * NI; ++n) dma(r0A, r0B, a, n);
    }
    wait_vm<kInFlight * 2 * NI>();
    lds_barrier();
    {
      i32x4_t r0A, r0B;
      stage_rsrc(ks0 + kSlots16 - 2, r0A, r0B);
#pragma unroll
      for (int n = 0; n < 2 * NI; ++n) dma(r0A, r0B, kSlots16 - 2, n);
    }
    typename Op16<T>::v4 op[2][8][2];             // [buffer][a0..a3, b0..b3][lo, hi]
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        op[0][f][h] = tr_at<T>((f < 4 ? ldsA + offA[f] : ldsB + offB[f - 4]) + h * 2048u);
    // Stages run in groups of kSlots16 with the ring slot a compile-time
    // constant, so every LDS address is a lane offset plus a constant that
    // folds into the instruction (no per-stage address arithmetic).
    auto stage = [&]<int SLOT>(int kk) {
      constexpr int NSLOT = (SLOT + 1) % kSlots16, DSLOT = (SLOT + kSlots16 - 1) % kSlots16;
      const uint32_t bA = ldsA + (uint32_t)SLOT * kSlotBytes, bB = ldsB + (uint32_t)SLOT * kSlotBytes;
      const uint32_t nA = ldsA + (uint32_t)NSLOT * kSlotBytes, nB = ldsB + (uint32_t)NSLOT * kSlotBytes;
      i32x4_t rnA, rnB;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        const bool last = (ks == NKS - 1);
        if (last) {
          wait_vm<kInFlight * 2 * NI>();
          lds_barrier();
          stage_rsrc(kk + kSlots16 - 1, rnA, rnB);
        }
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int i = n >> 2, j = n & 3;
          typename Op16<T>::v8 av, bv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            av[e] = op[cur][i][0][e]; av[e + 4] = op[cur][i][1][e];
            bv[e] = op[cur][4 + j][0][e]; bv[e + 4] = op[cur][4 + j][1][e];
          }
          acc[i][j] = Op16<T>::mfma(av, bv, acc[i][j]);
          const int f = n >> 1, h = n & 1;
          if (!last)
            op[nxt][f][h] = tr_at<T>((f < 4 ? bA + offA[f] : bB + offB[f - 4]) +
                                     (uint32_t)(ks + 1) * kSliceBytes + h * 2048u);
          else
            op[nxt][f][h] = tr_at<T>((f < 4 ? nA + offA[f] : nB + offB[f - 4]) + h * 2048u);
          if (last && (n & 1) == 0) dma(rnA, rnB, DSLOT, n >> 1);   // a copy every second MFMA
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    static_assert(kSlots16 == 5, "stage groups of five");
    int kk = ks0;                                  // stage kk uses slot (kk - ks0) % kSlots16
    for (; kk + 5 <= ks1; kk += 5) {
      if (((kk - ks0) / kSlots16) % kPaceEvery == 0) pace_at(done + (unsigned)(kk - ks0));
      stage.template operator()<0>(kk);
      stage.template operator()<1>(kk + 1);
      stage.template operator()<2>(kk + 2);
      stage.template operator()<3>(kk + 3);
      stage.template operator()<4>(kk + 4);
    }
    if (kk < ks1) stage.template operator()<0>(kk++);
    if (kk < ks1) stage.template operator()<1>(kk++);
    if (kk < ks1) stage.template operator()<2>(kk++);
    if (kk < ks1) stage.template operator()<3>(kk++);
  }
  if (PACE) done += (unsigned)(ks1 - ks0);

  if constexpr (UPD) {
    // The tile's row and column exponents go to LDS: the stage ring is free
    // once every wave is past its last stage and the copies issued ahead
    // (empty ones past the tile's end still write their zeros) have landed.
    int* eRow = reinterpret_cast<int*>(&sA[0][0]);
    int* eCol = eRow + kT16;
    wait_vm0();
    lds_barrier();
    {
      const int r = I * kT16 + tid, c = J * kT16 + tid;
      eRow[tid] = (r < d) ? piece_exp(up.sA[r]) : 0;
      eCol[tid] = (c < dB) ? piece_exp(up.sB[c]) : 0;
    }
    __syncthreads();
    // C + alpha 2^(eRow + eCol - 28) acc, 32 rows at a time.  Every load of a
    // group is issued before its stores (a load after a store through the
    // same pointer would wait for it), through a buffer resource at the
    // wave's block: one lane offset, the row offsets wave-uniform (scalar),
    // so 64 loads in flight need no address registers.
    if (cwrite) {
      const float sg = (MODE == 1 || up.neg) ? -1.0f : 1.0f;
      const bool rd = (MODE == 1) || up.beta;
      const int ldc = up.ldc;
      const __amdgpu_buffer_rsrc_t cr =
          __builtin_amdgcn_make_buffer_rsrc(up.C + (size_t)cm0 * ldc + cn0, (short)0, 0x7ffffff0, 0x00020000);
      const int vo = (4 * (lane >> 5) * ldc + (lane & 31)) * 4;
      // blocks wholly inside C take no per-element guard (MODE 1: always); the
      // guarded form (edge blocks of a ragged C) is a separate code path
      auto epi = [&]<bool G, bool RD>() {
#pragma unroll
        for (int ih = 0; ih < 4; ih += 1) {
          float old[1][4][16];
#pragma unroll
          for (int i2 = 0; i2 < 1; ++i2)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int i = ih + i2;
                const int so = ((i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32) * 4;
                old[i2][j][r] = 0.0f;
                if (RD && (!G || c_in(i, j, r)))
                  old[i2][j][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cr, vo, so, 0));
              }
#pragma unroll
          for (int i2 = 0; i2 < 1; ++i2)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int i = ih + i2;
                const int so = ((i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32) * 4;
                if (!G || c_in(i, j, r)) {
                  const int ex = eRow[wm * 128 + 4 * (lane >> 5) + i * 32 + 8 * (r >> 2) + (r & 3)] +
                                 eCol[wn * 128 + (lane & 31) + j * 32] - 28;
                  __builtin_amdgcn_raw_buffer_store_b32(
                      __builtin_bit_cast(uint32_t, old[i2][j][r] + sg * ldexpf(acc[i][j][r], ex)), cr, vo, so, 0);
                }
              }
        }
      };
      const bool whole = MODE == 1 || (cm0 + 128 <= d && cn0 + 128 <= dB);
      if (whole && rd)
        epi.template operator()<false, true>();
      else if (MODE == 2 && whole)
        epi.template operator()<false, false>();
      else if (MODE == 2 && rd)
        epi.template operator()<true, true>();
      else if (MODE == 2)
        epi.template operator()<true, false>();
    }
  } else if (up.C) {
    // One token split (up.C = H, row pitch d): no partial tile and no
    // reduction pass; the tile adds 2 acc into H itself (fl(H + 2 acc), the
    // same rounding as the reduction's) and, off the diagonal, into the
    // mirrored block.  Each 32-row group's loads are issued before its stores.
    if (cm0 < d && cn0 < d) {
      float* H = up.C;
      const __amdgpu_buffer_rsrc_t hr =
          __builtin_amdgcn_make_buffer_rsrc(H + (size_t)cm0 * d + cn0, (short)0, 0x7ffffff0, 0x00020000);
      const __amdgpu_buffer_rsrc_t mr =
          __builtin_amdgcn_make_buffer_rsrc(H + (size_t)cn0 * d + cm0, (short)0, 0x7ffffff0, 0x00020000);
      const int vo = (4 * (lane >> 5) * d + (lane & 31)) * 4;   // (row, col) of the block
      const int vm = ((lane & 31) * d + 4 * (lane >> 5)) * 4;   // (col, row): the mirror
      if (cm0 + 128 <= d && cn0 + 128 <= d) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          if (pass == 1 && I == J) break;
          const __amdgpu_buffer_rsrc_t br = pass ? mr : hr;
          const int vl = pass ? vm : vo;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float old[4][16];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int rr = i * 32 + 8 * (r >> 2) + (r & 3), cc = j * 32;
                const int so = (pass ? cc * d + rr : rr * d + cc) * 4;
                old[j][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, vl, so, 0));
              }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int rr = i * 32 + 8 * (r >> 2) + (r & 3), cc = j * 32;
                const int so = (pass ? cc * d + rr : rr * d + cc) * 4;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, old[j][r] + 2.0f * acc[i][j][r]),
                                                      br, vl, so, 0);
              }
          }
        }
      } else {
        // a block at the edge of H (d not a multiple of 128)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = cm0 + 4 * (lane >> 5) + i * 32 + 8 * (r >> 2) + (r & 3);
              const int col = cn0 + (lane & 31) + j * 32;
              if (row < d && col < d) {
                H[(size_t)row * d + col] += 2.0f * acc[i][j][r];
                if (I != J) H[(size_t)col * d + row] += 2.0f * acc[i][j][r];
              }
            }
      }
    }
  } else {
    float* out = partial + ((size_t)w * 4 + wave) * (16 * 16 * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) out[((i * 4 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  }
  }
  // finished: no one waits on this workgroup
  if (PACE && wave == 0 && lane == 0) __hip_atomic_store(prow + c, ~0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_32x32x2f32 (lane l supplies A[l%32][k=l/32]).
// Workgroup tile 128x128, 4 waves (2x2) of 64x64, 16 tokens per stage.
// ---------------------------------------------------------------------------
constexpr int kT32 = 128;
constexpr int kK32 = 16;
constexpr int kP32 = kT32 + 32;   // rows 32 banks apart: the two half-waves never collide

__global__ __launch_bounds__(256, 2) void syrk32_kernel(const float* __restrict__ X, int64_t n_tokens,
                                                         int d, int nt, int ntiles, int splits,
                                                         int64_t nk, float* __restrict__ partial,
                                                         double* __restrict__ pdiag) {
  __shared__ __attribute__((aligned(16))) float sA[2][kK32 * kP32];
  __shared__ __attribute__((aligned(16))) float sB[2][kK32 * kP32];
  __shared__ double sD[8][kT32 + 1];
  int s, I, J;
  if (!xcd_item(blockIdx.x, nt, ntiles, splits, s, I, J)) return;
  const int w = s * ntiles + tri_index(I, J);     // partial slot
  const bool diag = (I == J);
  const int64_t ks0 = nk * s / splits, ks1 = nk * (s + 1) / splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // 16 rows x 128 channels = 512 float4 per panel: 2 per thread
  const int crow = tid >> 5;          // 0..7 (+8)
  const int ccol = (tid & 31) * 4;
  const int chA = I * kT32 + ccol, chB = J * kT32 + ccol;
  const bool okA = chA < d, okB = chB < d;   // d % 8 == 0 => whole float4 in or out
  float4 ra[2], rb[2];
  auto gload = [&](int64_t kstep) {
    const int64_t t0 = kstep * kK32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t t = t0 + crow + 8 * i;
      const bool tv = t < n_tokens;
      ra[i] = (tv && okA) ? *reinterpret_cast<const float4*>(X + t * d + chA) : make_float4(0, 0, 0, 0);
      if (!diag)
        rb[i] = (tv && okB) ? *reinterpret_cast<const float4*>(X + t * d + chB) : make_float4(0, 0, 0, 0);
    }
  };
  double dsum[4] = {0.0, 0.0, 0.0, 0.0};
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<float4*>(&sA[buf][(crow + 8 * i) * kP32 + ccol]) = ra[i];
      if (!diag) *reinterpret_cast<float4*>(&sB[buf][(crow + 8 * i) * kP32 + ccol]) = rb[i];
    }
    if (diag) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float vv[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum[e] = fma((double)vv[e], (double)vv[e], dsum[e]);
      }
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (ks0 < ks1) {
    gload(ks0);
    lstore(0);
    __syncthreads();
    for (int64_t kk = ks0; kk < ks1; ++kk) {
      const int buf = (int)((kk - ks0) & 1);
      if (kk + 1 < ks1) gload(kk + 1);
      const float* stA = sA[buf];
      const float* stB = diag ? sA[buf] : sB[buf];
#pragma unroll
      for (int k2 = 0; k2 < kK32; k2 += 2) {
        const int row = (k2 + (lane >> 5)) * kP32;
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = stA[row + wm * 64 + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = stB[row + wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (kk + 1 < ks1) lstore(buf ^ 1);
      __syncthreads();
    }
  }
  float* out = partial + ((size_t)w * 4 + wave) * (4 * 16 * 64);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[((i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];

  if (diag) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sD[crow][ccol + e] = dsum[e];
    __syncthreads();
    if (tid < kT32) {
      double t = 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r) t += sD[r][tid];
      pdiag[((size_t)s * nt + I) * kT32 + tid] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// H += 2 * sum_s partial[s]  (fixed order), mirrored for off-diagonal tiles.
// One workgroup per (tile, wave sub-tile); WB = 32-blocks per sub-tile edge.
// ---------------------------------------------------------------------------
template <int WB, int NT>
__global__ __launch_bounds__(NT) void syrk_reduce_kernel(const float* __restrict__ partial,
                                                         float* __restrict__ H, int d, int ntiles,
                                                         int splits) {
  constexpr int E = 32 * WB;            // sub-tile edge
  constexpr int NEL = WB * WB * 1024;   // elements per wave sub-tile
  constexpr int NV = NEL / (4 * NT);    // float4 per thread
  constexpr int TILE = 2 * E;
  __shared__ float sub[E][E + 1];
  const int q = blockIdx.x >> 2, wave = blockIdx.x & 3;
  int I, J;
  tri_tile(q, I, J);
  const int row0 = I * TILE + (wave >> 1) * E;
  const int col0 = J * TILE + (wave & 1) * E;
  const size_t item_stride4 = (size_t)ntiles * 4 * NEL / 4;
  const float4* src = reinterpret_cast<const float4*>(partial + ((size_t)q * 4 + wave) * NEL);
  const int tid = threadIdx.x;
  // the splits are added in fp64 (in a fixed order) and rounded once
  double acc[NV][4];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0;
  for (int s = 0; s < splits; ++s) {
    const float4* ps = src + s * item_stride4;
    float4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ps[tid + NT * i];      // all loads in flight
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      acc[i][0] += v[i].x; acc[i][1] += v[i].y; acc[i][2] += v[i].z; acc[i][3] += v[i].w;
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float a4[4] = {(float)(2.0 * acc[i][0]), (float)(2.0 * acc[i][1]), (float)(2.0 * acc[i][2]),
                         (float)(2.0 * acc[i][3])};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * (tid + NT * i) + u;
      const int blk = e >> 10, r = (e >> 6) & 15, lane = e & 63;
      const int m = (blk / WB) * 32 + mfma32_row(r, lane);
      const int n = (blk % WB) * 32 + mfma32_col(lane);
      sub[m][n] = a4[u];
    }
  }
  __syncthreads();
  // H[row0 + m][col0 + n] += sub[m][n] (rows coalesced), then the mirror
  // H[col0 + n][row0 + m] += sub[m][n]; each batch of 16 reads is issued before
  // its 16 writes so the read-modify-writes do not serialize
  constexpr int NB = 16;
  for (int pass = 0; pass < ((I == J) ? 1 : 2); ++pass) {
    for (int e0 = 0; e0 < E * E; e0 += NT * NB) {
      float old[NB];
      size_t off[NB];
      bool ok[NB];
      float add[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = e0 + u * NT + tid;
        const int a = e / E, b = e % E;           // pass 0: (m, n) = (a, b); pass 1: (n, m)
        const int m = pass ? b : a, n = pass ? a : b;
        ok[u] = (e < E * E) && row0 + m < d && col0 + n < d;
        off[u] = pass ? (size_t)(col0 + n) * d + (row0 + m) : (size_t)(row0 + m) * d + (col0 + n);
        add[u] = ok[u] ? sub[m][n] : 0.0f;
        old[u] = ok[u] ? H[off[u]] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (ok[u]) H[off[u]] = old[u] + add[u];
    }
  }
}

// hdiag[c] += 2 * sum_s pdiag[s][c]   (fixed order, fp64)
__global__ __launch_bounds__(256) void diag_reduce_kernel(const double* __restrict__ pdiag, int d,
                                                          int np, int splits,
                                                          double* __restrict__ hdiag) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double t = 0.0;
  for (int s = 0; s < splits; ++s) t += pdiag[(size_t)s * np + c];
  hdiag[c] += 2.0 * t;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct SyrkPlan {
  int tile;       // 256 (16-bit inputs) or 128 (fp32)
  int ntiles;
  int splits;
  int64_t nk;     // number of token stages
  int nt;         // tile rows
  size_t off_diag;
  size_t off_pace;  // kXCD x kPaceSlots progress slots of the 16-bit kernel
  size_t off_sq;    // the 16-bit path's fp64 sums of squares [d] and their token-split partials
  size_t sq_ws;
  size_t ws;      // partial buffers, bytes
};

__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void zero_f64_kernel(double* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

// hdiag[c] += 2 * t[c]  (t: the channels' sums of squares)
__global__ __launch_bounds__(256) void add_twice_kernel(double* __restrict__ hdiag, const double* __restrict__ t, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) hdiag[i] += 2.0 * t[i];
}

static SyrkPlan syrk_plan(int64_t n_tokens, int d, bool f32, size_t max_ws = SIZE_MAX) {
  SyrkPlan p;
  p.tile = f32 ? kT32 : kT16;
  const int kst = f32 ? kK32 : kK16;
  const int nt = (d + p.tile - 1) / p.tile;
  p.nt = nt;
  p.ntiles = nt * (nt + 1) / 2;
  p.nk = (n_tokens + kst - 1) / kst;
  // Pick the split count that minimizes (rounds of 256 resident workgroups per
  // unit of work) plus the partial-sum traffic, with >= 16 stages per split.
  const double tile_flops = 2.0 * p.tile * p.tile * (double)kst;   // per stage
  const double t_stage = tile_flops / (2.5e15 / 256.0 * 0.6);      // s per stage per WG
  const double bytes_tile = (double)p.tile * p.tile * 4.0 * 2.0;    // partial write + read
  double best = 1e300;
  int best_s = 1;
  int smax = (int)std::max<int64_t>(1, std::min<int64_t>(64, p.nk / 16));
  // a scratch bound caps the split count (each split holds one partial per tile)
  const size_t per_split = (size_t)p.ntiles * p.tile * p.tile * sizeof(float) +
                           (f32 ? (size_t)nt * p.tile * sizeof(double) : 0) + 2 * kAlign +
                           (size_t)kXCD * kPaceSlots * sizeof(unsigned);
  if (max_ws != SIZE_MAX) smax = std::max(1, std::min<int>(smax, (int)(max_ws / per_split)));
  for (int s = 1; s <= smax; ++s) {
    const double items = (double)kXCD * ((p.ntiles + kXCD - 1) / kXCD) * s;
    const double rounds = std::ceil(items / 256.0);
    const double t = rounds * ((double)p.nk / s) * t_stage + items * bytes_tile / 6.0e12;
    if (t < best * 0.999) { best = t; best_s = s; }
  }
  p.splits = (p.nk == 0) ? 1 : best_s;
  const size_t per_item = (size_t)p.tile * p.tile * sizeof(float);
  p.off_diag = align_up((size_t)p.splits * p.ntiles * per_item);
  // fp64 diagonal partials: the fp32 kernel's (16-bit inputs sum x^2 in a pass of their own)
  p.off_pace = align_up(p.off_diag + (f32 ? (size_t)p.splits * nt * p.tile * sizeof(double) : 0));
  p.off_sq = align_up(p.off_pace + (size_t)kXCD * kPaceSlots * sizeof(unsigned));
  p.sq_ws = f32 ? 0 : gptq_awq_sumsq_workspace_size(n_tokens, d);
  p.ws = align_up(p.off_sq + (f32 ? 0 : align_up((size_t)d * sizeof(double)) + p.sq_ws));
  return p;
}

// The calls below share one launch sequence; ws holds the plan's partials.
static int hessian_launch(float* H, double* hdiag, const void* X, gptq_dtype x_dtype, int64_t n_tokens,
                          int32_t d_in, const SyrkPlan& p, void* ws, hipStream_t s) {
  const bool f32 = (x_dtype == GPTQ_F32);
  float* partial = static_cast<float*>(ws);
  double* pdiag = reinterpret_cast<double*>(static_cast<char*>(ws) + p.off_diag);
  unsigned* pace = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + p.off_pace);
  if (hdiag && !f32) {
    // the 16-bit path's fp64 keys come from one streaming pass over X (exact
    // squares summed in fp64, token splits added in a fixed order): summing
    // them inside the SYRK tiles cost ~9 % of the call, the pass ~1.5 %
    double* t = reinterpret_cast<double*>(static_cast<char*>(ws) + p.off_sq);
    void* sq_ws = static_cast<char*>(ws) + p.off_sq + align_up((size_t)d_in * sizeof(double));
    zero_f64_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(t, d_in);
    GPTQ_LAUNCH_CHECK();
    const int st = gptq_awq_act_sumsq(t, X, x_dtype, n_tokens, d_in, sq_ws, p.sq_ws, s);
    if (st != GPTQ_OK) return st;
    add_twice_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(hdiag, t, d_in);
    GPTQ_LAUNCH_CHECK();
  }
  const unsigned items = (unsigned)(kXCD * ((p.ntiles + kXCD - 1) / kXCD) * p.splits);
  // 16-bit path: one resident workgroup per CU (256 CUs), persistent over items
  const unsigned pgrid = std::min<unsigned>(256u, items);
  const unsigned pg = (pgrid + kXCD - 1) / kXCD * kXCD;
  // pacing (rare polls) for every 16-bit plan: at 8192 x 28672 (one split)
  // 197 -> 176 ms; with split token ranges 0-3 % (4096 .. 11008 columns)
  const bool pace_on = !f32;
  if (pace_on) {
    zero_u32_kernel<<<1, 256, 0, s>>>(pace, kXCD * kPaceSlots);
    GPTQ_LAUNCH_CHECK();
  }
  // one token split: the 16-bit tiles add into H themselves (no reduction)
  const bool direct = !f32 && p.splits == 1;
  Split3Args da{};
  if (direct) da.C = H;
  if (x_dtype == GPTQ_BF16) {
    auto k = pace_on ? syrk16_kernel<__bf16, true, 0> : syrk16_kernel<__bf16, false, 0>;
    k<<<pg, 256, 0, s>>>(static_cast<const __bf16*>(X), n_tokens, d_in, p.nt, p.ntiles, p.splits,
                         (int)p.nk, partial, pace, da);
  } else if (x_dtype == GPTQ_F16) {
    auto k = pace_on ? syrk16_kernel<_Float16, true, 0> : syrk16_kernel<_Float16, false, 0>;
    k<<<pg, 256, 0, s>>>(static_cast<const _Float16*>(X), n_tokens, d_in, p.nt, p.ntiles, p.splits,
                         (int)p.nk, partial, pace, da);
  } else {
    syrk32_kernel<<<items, 256, 0, s>>>(static_cast<const float*>(X), n_tokens, d_in, p.nt, p.ntiles,
                                        p.splits, p.nk, partial, pdiag);
  }
  GPTQ_LAUNCH_CHECK();
  if (f32)
    syrk_reduce_kernel<2, 256><<<p.ntiles * 4, 256, 0, s>>>(partial, H, d_in, p.ntiles, p.splits);
  else if (!direct)
    // 512 threads: the 66 KB LDS tile allows two workgroups per CU, so the
    // loads in flight come from more threads per workgroup
    syrk_reduce_kernel<4, 512><<<p.ntiles * 4, 512, 0, s>>>(partial, H, d_in, p.ntiles, p.splits);
  GPTQ_LAUNCH_CHECK();
  if (hdiag && f32) {
    diag_reduce_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(pdiag, d_in, p.nt * p.tile, p.splits, hdiag);
    GPTQ_LAUNCH_CHECK();
  }
  return GPTQ_OK;
}

static int hessian_check(float* H, const void* X, gptq_dtype x_dtype, int64_t n_tokens, int32_t d_in) {
  if (!H || d_in <= 0 || d_in > 65536 || (d_in % 8) != 0 || n_tokens < 0) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  if (!X || (reinterpret_cast<uintptr_t>(X) & 15)) return GPTQ_ERR_INVALID_ARG;
  return 1;
}

// ---------------------------------------------------------------------------
// The variant that allocates nothing: its partials live in this file-scope
// array, one copy per GPU, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): the
// device address is looked up once per device and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(256) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GPTQ_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GPTQ_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GPTQ_OK;
}

// ---------------------------------------------------------------------------
// Split products (the factor's super-block updates and the tree's large
// nodes, the column loop's super-block tails): scaled fp16 pieces of fp32
// operands on the update modes of the tile loop
// ---------------------------------------------------------------------------
// Largest |x| of each column c < n of a K x n panel (row pitch ld) as float
// bits, by atomicMax on the bits of non-negative floats (order-free); with
// `upper` only k <= c counts (an upper-triangular operand).  out starts at 0.
// A thread takes four adjacent columns (16-byte loads, n and ld multiples of
// 4) over 16 rows, eight rows' loads in flight.
__global__ __launch_bounds__(256) void col_absmax_kernel(const float* __restrict__ P, int ld, int K, int n, bool upper,
                                                         unsigned* __restrict__ out) {
  // a workgroup takes 256 columns by 64 rows: four row groups of 16 rows, one
  // wave each (a lane: four columns), their maxima combined in LDS before the
  // one atomic per column (the maximum is exact in any order)
  __shared__ float red[4][256];
  const int tx = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int c = blockIdx.x * 256 + tx * 4;
  const int k0 = blockIdx.y * 64 + rg * 16;
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (c < n) {
    const int k1 = min(K, upper ? min(k0 + 16, c + 4) : k0 + 16);
    for (int k = k0; k < k1; k += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = (k + u < k1) ? *reinterpret_cast<const float4*>(P + (size_t)(k + u) * ld + c) : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float a[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (!upper || k + u <= c + q) m[q] = fmaxf(m[q], fabsf(a[q]));
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) red[rg][tx * 4 + q] = m[q];
  __syncthreads();
  if (rg == 0 && c < n) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = tx * 4 + q;
      const float mm = fmaxf(fmaxf(red[0][j], red[1][j]), fmaxf(red[2][j], red[3][j]));
      if (mm > 0.0f) atomicMax(out + c + q, __builtin_bit_cast(unsigned, mm));
    }
  }
}

// Largest |A[i][k]| of each row i < m of a row-major m x K matrix (pitch
// lda), one workgroup per row; with `upper` only k >= i counts.
__global__ __launch_bounds__(256) void row_absmax_kernel(const float* __restrict__ A, int lda, int K, bool upper,
                                                         unsigned* __restrict__ out) {
  __shared__ float red[4];
  const int i = blockIdx.x, tid = threadIdx.x;
  float m = 0.0f;
  for (int k = (upper ? i : 0) + tid; k < K; k += 256) m = fmaxf(m, fabsf(A[(size_t)i * lda + k]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) out[i] = __builtin_bit_cast(unsigned, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

// the two fp16 pieces of x scaled by 2^(14 - e)
GPTQ_DEV void split2(float x, int e, _Float16& h, _Float16& l) {
  const float xs = ldexpf(x, 14 - e);
  h = (_Float16)xs;
  l = (_Float16)(xs - (float)h);
}

// planes[p][k][c] (row pitch n), p = 0, 1: h, l of P[k][c] scaled by its
// column's exponent (smax[c]); with `upper` entries below P's diagonal
// (k > c) are taken as zero.
__global__ __launch_bounds__(256) void split3_planes_kernel(const float* __restrict__ P, int ldp, int K, int n,
                                                            const unsigned* __restrict__ smax, bool upper,
                                                            _Float16* __restrict__ planes) {
  const int64_t total = (int64_t)K * n;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= total) return;
  const int k = (int)(e / n), c = (int)(e - (int64_t)k * n);
  const float4 v = *reinterpret_cast<const float4*>(P + (size_t)k * ldp + c);
  const float a[4] = {v.x, v.y, v.z, v.w};
  f16x4_t h, l;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float x = (upper && k > c + u) ? 0.0f : a[u];
    _Float16 hu, lu;
    split2(x, piece_exp(smax[c + u]), hu, lu);
    h[u] = hu;
    l[u] = lu;
  }
  *reinterpret_cast<f16x4_t*>(planes + e) = h;
  *reinterpret_cast<f16x4_t*>(planes + total + e) = l;
}

// planes[p][k][i] (row pitch m), p = 0, 1: h, l of A[i][k] for A m x K
// row-major (pitch lda), scaled by its row's exponent (smax[i]), transposed
// through a 64 x 64 LDS tile; with `upper` the entries below A's diagonal
// (k < i) are taken as zero.
__global__ __launch_bounds__(256) void split3_planes_t_kernel(const float* __restrict__ A, int lda, int K, int m,
                                                              const unsigned* __restrict__ smax, bool upper,
                                                              _Float16* __restrict__ planes) {
  __shared__ float t[64][65];
  const int k0 = blockIdx.x * 64, i0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, r = e >> 4, c4 = (e & 15) * 4;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (i0 + r < m && k0 + c4 < K) v = *reinterpret_cast<const float4*>(A + (size_t)(i0 + r) * lda + k0 + c4);
    t[r][c4] = v.x;
    t[r][c4 + 1] = v.y;
    t[r][c4 + 2] = v.z;
    t[r][c4 + 3] = v.w;
  }
  __syncthreads();
  const int64_t total = (int64_t)K * m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, rr = e >> 4, cc = (e & 15) * 4;
    const int k = k0 + rr, i = i0 + cc;
    if (k >= K || i >= m) continue;
    f16x4_t h, l;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x = (upper && k < i + u) ? 0.0f : t[cc + u][rr];
      _Float16 hu, lu;
      split2(x, piece_exp(smax[i + u]), hu, lu);
      h[u] = hu;
      l[u] = lu;
    }
    const int64_t o = (int64_t)k * m + i;
    *reinterpret_cast<f16x4_t*>(planes + o) = h;
    *reinterpret_cast<f16x4_t*>(planes + total + o) = l;
  }
}

// The split form runs 256 resident 256 x 256 tiles per round at about 1 PFLOP/s
// of fp16 products, three per fp32 product; the fp32 tiles reach ~110 TFLOP/s.
// From one round of tiles on (n ~ 5600) it is the faster of the two
// (measured at d = 13824: 528 -> 256 tiles, prepare 16.7 -> 16.1 ms).
bool split3_pays(int n) {
  const int nt = (n + kT16 - 1) / kT16;
  return nt * (nt + 1) / 2 >= 256;
}

// planes (h, l: 2 K n fp16), then the columns' largest |x| (n u32)
size_t split3_planes_bytes(int K, int n) { return align_up(4 * (size_t)K * n) + align_up(4 * (size_t)n); }

int split3_update(const float* P, int ldp, int K, int n, float* C, int ldc, void* planes, hipStream_t s) {
  if (!P || !C || !planes || K <= 0 || K % kK16 != 0 || n <= 0 || n % 128 != 0 || ldp % 4 != 0 || ldp < n ||
      ldc < n || (size_t)K * kSegs / kK16 > (size_t)INT32_MAX)
    return GPTQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(P) % 16 != 0 || reinterpret_cast<uintptr_t>(planes) % 16 != 0)
    return GPTQ_ERR_INVALID_ARG;
  _Float16* pl = static_cast<_Float16*>(planes);
  const int64_t total = (int64_t)K * n;
  unsigned* smax = reinterpret_cast<unsigned*>(static_cast<char*>(planes) + align_up(4 * (size_t)total));
  zero_u32_kernel<<<1, 256, 0, s>>>(smax, n);
  GPTQ_LAUNCH_CHECK();
  col_absmax_kernel<<<dim3((n + 255) / 256, (K + 63) / 64), 256, 0, s>>>(P, ldp, K, n, false, smax);
  GPTQ_LAUNCH_CHECK();
  split3_planes_kernel<<<(unsigned)((total / 4 + 255) / 256), 256, 0, s>>>(P, ldp, K, n, smax, false, pl);
  GPTQ_LAUNCH_CHECK();
  const int nt = (n + kT16 - 1) / kT16, ntiles = nt * (nt + 1) / 2;
  const unsigned items = (unsigned)(kXCD * ((ntiles + kXCD - 1) / kXCD));
  const unsigned pg = (std::min<unsigned>(256u, items) + kXCD - 1) / kXCD * kXCD;
  Split3Args a{};
  a.C = C;
  a.ldc = ldc;
  a.kseg = K;
  a.plane = total;
  a.sA = smax;
  a.sB = smax;
  syrk16_kernel<_Float16, false, 1><<<pg, 256, 0, s>>>(pl, (int64_t)kSegs * K, n, nt, ntiles, 1, kSegs * K / kK16,
                                                       nullptr, nullptr, a);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

// The general form pays from half a round of 256 x 256 tiles on (the tree's
// nodes of 3456 x 3456 at d = 13824 among them).
bool split3_gemm_shape_ok(int K, int m, int n) {
  if (K <= 0 || K % kK16 != 0 || m <= 0 || n <= 0 || m % 8 != 0 || n % 8 != 0) return false;
  if ((size_t)K * kSegs / kK16 > (size_t)INT32_MAX) return false;
  const int64_t tiles = (int64_t)((m + kT16 - 1) / kT16) * ((n + kT16 - 1) / kT16);
  return tiles >= 128;
}

bool split3_gemm_applies(const float* A, int lda, bool a_rows, const float* B, int ldb, int K, int m, int n) {
  if (!A || !B || !split3_gemm_shape_ok(K, m, n)) return false;
  if (lda % 4 != 0 || ldb % 4 != 0 || lda < (a_rows ? K : m) || ldb < n) return false;
  return reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(B) % 16 == 0;
}

// planes of A and B (h, l: 2 K (m + n) fp16), then the largest |x| of A's
// rows of C and of B's columns (m + n u32)
size_t split3_gemm_planes_bytes(int K, int m, int n) {
  return align_up(4 * (size_t)K * ((size_t)m + (size_t)n)) + align_up(4 * ((size_t)m + (size_t)n)) +
         (size_t)kXCD * 32 * sizeof(unsigned);
}

int split3_gemm(const float* A, int lda, bool a_rows, const float* B, int ldb, int K, int m, int n, float* C,
                int ldc, bool neg, bool beta, int tri, void* planes, hipStream_t s) {
  if (!split3_gemm_applies(A, lda, a_rows, B, ldb, K, m, n) || !C || ldc < n || !planes ||
      reinterpret_cast<uintptr_t>(planes) % 16 != 0 || tri < 0 || tri > 2 || (tri == 1 && !a_rows))
    return GPTQ_ERR_INVALID_ARG;
  _Float16* pa = static_cast<_Float16*>(planes);
  const int64_t ta = (int64_t)K * m, tb = (int64_t)K * n;
  _Float16* pb = pa + 2 * ta;   // 2 K m elements: 16-byte aligned since m % 8 == 0
  unsigned* sA = reinterpret_cast<unsigned*>(static_cast<char*>(planes) + align_up(4 * (size_t)(ta + tb)));
  unsigned* sB = sA + m;
  zero_u32_kernel<<<1, 256, 0, s>>>(sA, m + n);
  GPTQ_LAUNCH_CHECK();
  if (a_rows)
    row_absmax_kernel<<<m, 256, 0, s>>>(A, lda, K, tri == 1, sA);
  else
    col_absmax_kernel<<<dim3((m + 255) / 256, (K + 63) / 64), 256, 0, s>>>(A, lda, K, m, false, sA);
  GPTQ_LAUNCH_CHECK();
  col_absmax_kernel<<<dim3((n + 255) / 256, (K + 63) / 64), 256, 0, s>>>(B, ldb, K, n, tri == 2, sB);
  GPTQ_LAUNCH_CHECK();
  if (a_rows)
    split3_planes_t_kernel<<<dim3((K + 63) / 64, (m + 63) / 64), 256, 0, s>>>(A, lda, K, m, sA, tri == 1, pa);
  else
    split3_planes_kernel<<<(unsigned)((ta / 4 + 255) / 256), 256, 0, s>>>(A, lda, K, m, sA, false, pa);
  GPTQ_LAUNCH_CHECK();
  split3_planes_kernel<<<(unsigned)((tb / 4 + 255) / 256), 256, 0, s>>>(B, ldb, K, n, sB, tri == 2, pb);
  GPTQ_LAUNCH_CHECK();
  const int mt = (m + kT16 - 1) / kT16, ntn = (n + kT16 - 1) / kT16, ntiles = mt * ntn;
  const unsigned items = (unsigned)(kXCD * ((ntiles + kXCD - 1) / kXCD));
  const unsigned pg = (std::min<unsigned>(256u, items) + kXCD - 1) / kXCD * kXCD;
  Split3Args a{};
  a.C = C;
  a.ldc = ldc;
  a.kseg = K;
  a.plane = ta;
  a.B = pb;
  a.planeB = tb;
  a.sA = sA;
  a.sB = sB;
  a.n = n;
  a.ntn = ntn;
  a.neg = neg ? 1 : 0;
  a.beta = beta ? 1 : 0;
  a.kmode = tri;
  if (tri != 0) {
    a.queue = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(sA) + align_up(4 * ((size_t)m + (size_t)n)));
    zero_u32_kernel<<<1, 256, 0, s>>>(a.queue, kXCD * 32);
    GPTQ_LAUNCH_CHECK();
  }
  syrk16_kernel<_Float16, false, 2><<<pg, 256, 0, s>>>(pa, (int64_t)kSegs * K, m, mt, ntiles, 1, kSegs * K / kK16,
                                                       nullptr, nullptr, a);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_workspace_size(int64_t n_tokens, int32_t d_in) {
  if (n_tokens < 0 || d_in <= 0) return 0;
  SyrkPlan a = syrk_plan(n_tokens, d_in, false), b = syrk_plan(n_tokens, d_in, true);
  return std::max(a.ws, b.ws);
}

extern "C" int gptq_hessian_accumulate(float* H, double* hdiag, const void* X, gptq_dtype x_dtype,
                                       int64_t n_tokens, int32_t d_in, void* ws, size_t ws_bytes,
                                       hipStream_t s) {
  const int c = hessian_check(H, X, x_dtype, n_tokens, d_in);
  if (c != 1) return c;
  const SyrkPlan p = syrk_plan(n_tokens, d_in, x_dtype == GPTQ_F32);
  if (!ws || ws_bytes < p.ws || ws_bytes < gptq_hessian_workspace_size(n_tokens, d_in))
    return GPTQ_ERR_WORKSPACE;
  return hessian_launch(H, hdiag, X, x_dtype, n_tokens, d_in, p, ws, s);
}

extern "C" size_t gptq_hessian_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int gptq_hessian_accumulate_noalloc(float* H, double* hdiag, const void* X,
                                               gptq_dtype x_dtype, int64_t n_tokens, int32_t d_in,
                                               hipStream_t s) {
  const int c = hessian_check(H, X, x_dtype, n_tokens, d_in);
  if (c != 1) return c;
  const SyrkPlan p = syrk_plan(n_tokens, d_in, x_dtype == GPTQ_F32, kScratchBytes);
  if (p.ws > kScratchBytes) return GPTQ_ERR_WORKSPACE;   // one split's partials do not fit
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st != GPTQ_OK) return st;
  return hessian_launch(H, hdiag, X, x_dtype, n_tokens, d_in, p, ws, s);
}
