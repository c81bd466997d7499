// layout.hpp -- device layout of a packed ARCHead head on gfx950.
//
// The packed module of the ARCHead paper (section 3.3) registers the SC4
// INT4 residual with its fp16 group scales, the 5-bit / 8-bit core factors
// with their scales, and the INT8 correction factors.  This file fixes how
// those fields sit in HBM so that the vocabulary-tile kernels read them with
// fully coalesced 16-byte loads and need no shuffles to feed MFMA.
//
// Vocabulary rows are grouped in blocks of 16 ("v-blocks"); the hidden
// dimension in K-steps of 32.  One K-step of one v-block is exactly the
// B operand of a v_mfma_f32_16x16x32 instruction: lane l (0..63) holds row
// (l % 16) of the block and the 8 consecutive columns 8*(l/16) .. +7 of the
// K-step.  Every field below stores, per (v-block, K-step), 64 lanes' worth
// of that operand back to back.
//
//  r4   uint32 [d/128][nvb][64][4]   SC4 residual, K-chunk major: for one
//       K-chunk the 1 KiB blocks of consecutive v-blocks are adjacent, so the
//       waves streaming neighbouring v-blocks read one contiguous region at a
//       time (v-block major order, with each wave's streams 32 KiB apart,
//       measured about 1.5x slower on MI355X).  Dword s of lane l in
//       K-chunk c covers columns 128c + 32s + 8(l/16) + e, e = 0..7; value
//       e sits in nibble (e>>1) + 4(e&1) as offset binary (q + 8).  Masking
//       nibbles (p, p+4) with 0x000F000F therefore yields the column pair
//       (2p, 2p+1) in the two 16-bit halves, in order.
//  sr   uint16 [nvb][G][16]          fp16 residual scales, G = d/g.
//  lr   uint32 [n_lr][nvb][64][4]   the low-rank codes (5-bit core factor A5
//       and INT8 correction factor C8) as a stream of 1 KiB v-block chunks,
//       K-chunk major like r4, so that the streaming kernel reads them through
//       the same pipeline as the residual.  kst = ceil(k/32), rst = ceil(r/32).
//       Chunks j = 0 .. na-1 (na = ceil(kst/3)) hold core K-steps 3j+q,
//       q = 0..2: dword q = low 4 bits of (a + 16) in the nibble order of r4,
//       dword 3 = bit 4 of (a + 16), for K-step q and column pair p, half h,
//       at bit (4 + 4q + p + 16h) mod 32, so rotating it right by 4q + p
//       lands the pair's two bits at positions 4 and 20.  Chunks na + j hold
//       correction K-steps 2j and 2j+1: dwords (0,1) and (2,3) = the lane's 8
//       columns as offset-binary bytes (c ^ 0x80) in natural order.  The chunk
//       count n_lr is padded to a multiple of 4; K-steps beyond kst / rst hold
//       the code of zero and are skipped.
//  srp  uint16 [nvb][G][16]          sR * 2^(e_r + 14) in fp16, an exact
//       power-of-two rescale with e_r per row such that the row's largest
//       residual scale lies in [2^14, 2^15); the large-M kernel turns each
//       code q into the fp16 value q sR 2^(e_r - 10) with one fused
//       multiply-add.
//  rsc  float  [nvb*16]              2^(10 - e_r) per row.
//  sa, sc  uint16 [nvb*16]           fp16 row scales of A5 and C8.
//  b8   int8   [k][d], sb float [k]  right core factor and its row scales.
//  d8   int8   [r][d], sd float [r][G]  quantised B_w and its group scales.
// Padding rows (v >= V) and padding columns (k..kst*32, r..rst*32) hold the
// code of zero with zero scales.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace archead {

constexpr int kVB = 16;      // vocabulary rows per v-block
constexpr int kKStep = 32;   // K columns per MFMA K-step
constexpr int kKChunk = 128; // K columns per 16-byte lane load of r4

struct Shape {
    int64_t V, d, k, r, g;
    __host__ __device__ int64_t nvb() const { return (V + kVB - 1) / kVB; }
    __host__ __device__ int64_t G() const { return d / g; }
    __host__ __device__ int64_t nkc() const { return d / kKChunk; }
    __host__ __device__ int64_t kst() const { return (k + kKStep - 1) / kKStep; }
    __host__ __device__ int64_t rst() const { return (r + kKStep - 1) / kKStep; }
    __host__ __device__ int64_t kpad() const { return kst() * kKStep; }
    __host__ __device__ int64_t rpad() const { return rst() * kKStep; }
    __host__ __device__ int64_t lr_na() const { return (kst() + 2) / 3; }  // A5 chunks
    __host__ __device__ int64_t lr_nc() const { return (rst() + 1) / 2; }  // C8 chunks
    // total low-rank chunks, rounded up to a multiple of 4 so that the
    // residual chunks start in the first of the prefetch buffers in both the
    // one- and the two-chunk pipelines (pad chunks are correction chunks
    // whose K-steps all lie beyond rst)
    __host__ __device__ int64_t n_lr() const { return (lr_na() + lr_nc() + 3) / 4 * 4; }

    // element counts of each device array
    __host__ __device__ size_t n_r4() const { return (size_t)nkc() * nvb() * 64 * 4; }      // uint32
    __host__ __device__ size_t n_sr() const { return (size_t)nvb() * G() * kVB; }           // uint16
    __host__ __device__ size_t n_rows() const { return (size_t)nvb() * kVB; }               // sa, sc
    __host__ __device__ size_t n_lr_words() const { return (size_t)n_lr() * nvb() * 64 * 4; } // uint32
};

// Raw device pointers of one loaded head (all device memory).
struct DevHead {
    Shape s;
    int n_cu; // compute units of the device the head lives on
    const uint32_t *r4;
    const uint16_t *sr;
    const uint32_t *lr;
    const uint16_t *srp;
    const float *rsc;
    const uint16_t *sa;
    const uint16_t *sc;
    const int8_t *b8;
    const float *sb;
    const int8_t *d8;
    const float *sd;
};

// Per-call workspace, written by the projection kernel and read by the
// vocabulary-tile kernels.  Mp = M rounded up to a multiple of 32.
struct Work {
    int64_t M, Mp;
    uint16_t *t16;     // [2][Mp][kpad] bf16 hi/lo of t = X (sB o B8)^T
    uint16_t *s16;     // [2][Mp][rpad] bf16 hi/lo of s = X (sD o D8)^T
    float *xsneg;      // [G][Mp]  -136 * sum_{j in group} X[m, j]
    // large-M path (Mq = M rounded up to 128):
    float *tf32;       // [Mp][kpad] t in fp32
    float *sf32;       // [Mp][rpad] s in fp32
    uint16_t *xsw;     // [Mq/16][d/32][64][8]    fp16 X 2^f_m in MFMA A-operand blocks
    uint16_t *tsw;     // [Mq/16][kst][2][64][8]  fp16 hi/lo of t 2^f_m, same blocks
    uint16_t *ssw;     // [Mq/16][rst][2][64][8]  fp16 hi/lo of s 2^f_m
    float *xsc;        // [Mq][2]  (2^-f_m, 2^f_m)
    int32_t *lfill;    // [stages][16]  what each stage of the large-M kernel copies
    int64_t Mq;
    uint64_t *part;    // [M][n_part] argmax partial keys
    int64_t n_part;
    int64_t part_cap;  // uint64 slots in part
    // single-launch decode path: work counters and argmax keys (layout
    // below), all zero between calls (the launch puts them back to zero)
    uint32_t *sync;    // [kSyncWords]
    uint64_t *keys;    // [kKeyWords]
    uint32_t *colflag; // [k + r] call number + 1 once column i of t / s is published
    // log-normaliser and cross-entropy of the logits (per call):
    int want_lse;           // write (max, sum exp) summaries beside the argmax keys
    const int32_t *targets; // [M] target row per hidden state, may be null
    uint64_t *lsep;         // [M][n_part] summaries (LsePart as 64 bits); the
                            // single-launch path uses [M][workgroups]
    float *tl;              // [M] the logit of each hidden state's target row
    // top-k selection: per (row, 1024-logit slice) the slice's K largest keys
    uint64_t *tkp;          // [M][slices][K]
    int64_t tkp_cap;        // uint64 slots in tkp
    // matrix-core projection for 5 <= M <= 32: per (16-column tile, K-slice)
    // partial sums, and per tile a count of slices done (zero between calls)
    float *ppart;           // [tiles][kProjKS][2][64][4]
    uint32_t *pcnt;         // [tiles]
};

constexpr int kProjKS = 8; // K-slices of the matrix-core projection for 5 <= M <= 32

constexpr int kDecodeMaxM = 2; // largest M of the single-launch decode path

// Work counters of the single-launch decode path.  Atomics on one address
// serialise (about 10 ns each), so counters that many workgroups update are
// split into kSyncGroups copies, each in its own 256-byte line:
//   (line g < kSyncGroups: unused)
//   slot_done[s]  workgroups of slot s finished
//   epoch         calls completed (never reset; tags the column flags)
//   top_done      slots finished
//   published     projection columns published (never reset: k + r per call)
// and the argmax keys: per slot s, keys[s * 32 + m], m < kDecodeMaxM.
constexpr int kSyncGroups = 16;
constexpr int kSyncStride = 64; // uint32 per 256-byte line
constexpr size_t kSyncWords = size_t(2 * kSyncGroups + 3) * kSyncStride;
constexpr size_t kKeyWords = size_t(kSyncGroups) * 32;
__host__ __device__ constexpr size_t sync_slot_done(int s) { return size_t(kSyncGroups + s) * kSyncStride; }
__host__ __device__ constexpr size_t sync_epoch() { return size_t(2 * kSyncGroups) * kSyncStride; }
__host__ __device__ constexpr size_t sync_top_done() { return size_t(2 * kSyncGroups + 1) * kSyncStride; }
__host__ __device__ constexpr size_t sync_published() { return size_t(2 * kSyncGroups + 2) * kSyncStride; }

// Host relayout (pack.cpp).  Inputs in the canonical host layout; outputs are
// host buffers in the device layout, sized by Shape::n_*.
struct HostDevImage {
    uint32_t *r4;
    uint16_t *sr;
    uint32_t *lr;
    uint16_t *srp;
    float *rsc;
    uint16_t *sa;
    uint16_t *sc;
    float *sb;
    float *sd;
};

void relayout(const Shape &s, const int8_t *A5, const uint16_t *sA, const uint16_t *sB,
              const uint8_t *R4, const uint16_t *sR, const int8_t *C8, const uint16_t *sC,
              const uint16_t *sD, const HostDevImage &out, int n_threads);

float half_to_float(uint16_t h);
uint16_t float_to_half(float f); // round to nearest even

} // namespace archead
