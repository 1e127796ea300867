// Internal definitions shared by the host planner (plan.cpp, no HIP) and the
// HIP launchers.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "sketchssm.h"

namespace skssm {

constexpr int kK = 128;         // key dim the kernels are written for
constexpr int kW = 16;          // window length (one MFMA M-tile of tokens)
constexpr int kMaxHeads = 256;  // head index fits a byte
constexpr int kMaxRank = 64;    // four 16-row MFMA tiles of sketch rows

// Per-launch-position head table, passed to the kernels by value (no device
// allocation is ever needed for it).  Entry p describes head order[p].
struct HeadTable {
    uint8_t head[kMaxHeads];
    uint8_t rank[kMaxHeads];    // 0 = dense fallback
    uint8_t group[kMaxHeads];
    uint32_t frow[kMaxHeads];   // first row of the head's frame in the frames array
    uint32_t zrow[kMaxHeads];   // z_row_off of the head
};

sketchssm_status check_shape(const sketchssm_shape* s);
// Table listing heads 0..H-1 in order, all dense (the full-state-read baseline).
void dense_table(const sketchssm_shape& s, HeadTable* t);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// key/query heads of a (checked) shape: kq_heads, or H when it is 0
inline int kq_heads_of(const sketchssm_shape& s) { return s.kq_heads > 0 ? s.kq_heads : s.H; }

}  // namespace skssm

struct sketchssm_plan {
    sketchssm_shape shape;
    std::vector<int32_t> rank, group;
    std::vector<int32_t> frame_index, frame_row_off, z_row_off, bucket, order;
    std::vector<int32_t> frame_group, frame_rank;
    int32_t n_frames = 0;
    int32_t n_dense = 0;     // dense heads come first in the order
    int32_t max_rank = 0;    // largest rank of any head
    size_t z_elems = 0;
    size_t frame_elems = 0;
    skssm::HeadTable table;
};
