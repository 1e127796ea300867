// Host planner: shape checks and the derivation of frames, offsets, buckets and
// the launch order from a per-head rank table.  Plain C++, no HIP calls, so it
// runs (and is tested) on machines without a GPU.
//
// On the calibration card ("SketchSSM calibration: Nemotron Nano 9B v2", opening
// paragraph) each head's rank and the order of the frames come out of the
// calibration's allocation scores for whatever mean rank is requested; the
// PyPI page ("Make a calibration for your model", allocate stage) gives each
// head a rank or a dense fallback, and the card caps ranks ("Contents":
// allocation rank cap 49).  The pages do not define the frame order or any
// scheduling; the rule here is this library's:
//   frames  = distinct (group, rank) of sketch heads, sorted by group then rank
//   bucket  = 0 for dense, else 1 + (rank - 1) / 8
//   order   = dense heads, then buckets high to low, head ascending inside one.
#include <algorithm>
#include <cstring>
#include <new>
#include <utility>

#include "sketchssm_internal.h"

namespace skssm {

sketchssm_status check_shape(const sketchssm_shape* s) {
    if (!s) return SKSSM_EINVAL;
    if (s->kind < SKSSM_MAMBA2 || s->kind > SKSSM_KDA) return SKSSM_EINVAL;
    if (s->qkv != SKSSM_BF16 && s->qkv != SKSSM_F32) return SKSSM_EINVAL;
    if (s->B < 1 || s->H < 1 || s->H > kMaxHeads) return SKSSM_ESHAPE;
    if (s->K != kK || s->W != kW) return SKSSM_ESHAPE;
    if (s->V < 64 || s->V > 128 || s->V % 16 != 0) return SKSSM_ESHAPE;
    if (s->G < 1 || s->G > kMaxHeads) return SKSSM_ESHAPE;
    if (s->basis_rows < 1 || s->rank_cap < 1 || s->rank_cap > kMaxRank) return SKSSM_ESHAPE;
    if (s->kq_heads < 0 || s->kq_heads > s->H || (s->kq_heads > 0 && s->H % s->kq_heads != 0))
        return SKSSM_ESHAPE;
    // every index used by the kernels stays below 2^31 elements per array
    const double sz = double(s->B) * s->H * s->K * s->V;
    if (sz >= 2147483648.0) return SKSSM_ESHAPE;
    return SKSSM_OK;
}

void dense_table(const sketchssm_shape& s, HeadTable* t) {
    std::memset(t, 0, sizeof(*t));
    for (int h = 0; h < s.H; ++h) t->head[h] = static_cast<uint8_t>(h);
}

}  // namespace skssm

using namespace skssm;

// The plan of a rank table; `order` (may be null) replaces the derived launch
// order: a permutation of 0..H-1 that lists every dense head before any sketch
// head (the read kernel's blocks take the dense heads first).
static sketchssm_status make_plan(const sketchssm_shape* shape, const int32_t* rank,
                                  const int32_t* group, const int32_t* order, sketchssm_plan** out) {
    if (!out) return SKSSM_EINVAL;
    *out = nullptr;
    if (!rank || !group) return SKSSM_EINVAL;
    sketchssm_status st = check_shape(shape);
    if (st != SKSSM_OK) return st;
    const int H = shape->H;
    const int rmax = std::min(std::min(shape->rank_cap, shape->basis_rows), shape->K);
    for (int h = 0; h < H; ++h) {
        if (group[h] < 0 || group[h] >= shape->G) return SKSSM_ESHAPE;
        if (rank[h] < 0 || rank[h] > rmax) return SKSSM_ESHAPE;
    }
    sketchssm_plan* p = new (std::nothrow) sketchssm_plan();
    if (!p) return SKSSM_ENOMEM;
    try {
        p->shape = *shape;
        p->rank.assign(rank, rank + H);
        p->group.assign(group, group + H);

        std::vector<std::pair<int32_t, int32_t>> fr;
        for (int h = 0; h < H; ++h)
            if (rank[h] > 0) fr.emplace_back(group[h], rank[h]);
        std::sort(fr.begin(), fr.end());
        fr.erase(std::unique(fr.begin(), fr.end()), fr.end());
        p->n_frames = static_cast<int32_t>(fr.size());
        p->frame_row_off.assign(1, 0);
        for (auto& f : fr) {
            p->frame_group.push_back(f.first);
            p->frame_rank.push_back(f.second);
            p->frame_row_off.push_back(p->frame_row_off.back() + f.second);
        }
        p->frame_index.assign(H, -1);
        p->z_row_off.assign(1, 0);
        p->bucket.assign(H, 0);
        for (int h = 0; h < H; ++h) {
            if (rank[h] > 0) {
                auto it = std::lower_bound(fr.begin(), fr.end(), std::make_pair(group[h], rank[h]));
                p->frame_index[h] = static_cast<int32_t>(it - fr.begin());
                p->bucket[h] = 1 + (rank[h] - 1) / 8;
            }
            p->z_row_off.push_back(p->z_row_off.back() + rank[h]);
            p->max_rank = std::max(p->max_rank, rank[h]);
        }
        p->order.resize(H);
        if (order) {
            p->order.assign(order, order + H);
        } else {
            for (int h = 0; h < H; ++h) p->order[h] = h;
            const std::vector<int32_t>& bk = p->bucket;
            std::stable_sort(p->order.begin(), p->order.end(), [&](int32_t x, int32_t y) {
                const bool dx = bk[x] == 0, dy = bk[y] == 0;
                if (dx != dy) return dx;          // dense first
                if (bk[x] != bk[y]) return bk[x] > bk[y];
                return x < y;
            });
        }
        p->n_dense = 0;
        for (int h = 0; h < H; ++h) p->n_dense += (rank[h] == 0);
        p->z_elems = size_t(shape->B) * shape->V * size_t(p->z_row_off.back());
        p->frame_elems = size_t(shape->K) * size_t(p->frame_row_off.back());

        std::memset(&p->table, 0, sizeof(p->table));
        for (int i = 0; i < H; ++i) {
            const int h = p->order[i];
            p->table.head[i] = static_cast<uint8_t>(h);
            p->table.rank[i] = static_cast<uint8_t>(rank[h]);
            p->table.group[i] = static_cast<uint8_t>(group[h]);
            p->table.frow[i] = rank[h] ? static_cast<uint32_t>(p->frame_row_off[p->frame_index[h]]) : 0u;
            p->table.zrow[i] = static_cast<uint32_t>(p->z_row_off[h]);
        }
    } catch (...) {
        delete p;
        return SKSSM_ENOMEM;
    }
    *out = p;
    return SKSSM_OK;
}

extern "C" sketchssm_status sketchssm_plan_create(const sketchssm_shape* shape, const int32_t* rank,
                                                  const int32_t* group, sketchssm_plan** out) {
    return make_plan(shape, rank, group, nullptr, out);
}

extern "C" sketchssm_status sketchssm_plan_create_ordered(const sketchssm_shape* shape,
                                                          const int32_t* rank, const int32_t* group,
                                                          const int32_t* order, sketchssm_plan** out) {
    if (!out) return SKSSM_EINVAL;
    *out = nullptr;
    if (!order || !rank) return SKSSM_EINVAL;
    const sketchssm_status st = check_shape(shape);
    if (st != SKSSM_OK) return st;
    const int H = shape->H;
    std::vector<char> seen(H, 0);
    bool sketch_seen = false;
    for (int i = 0; i < H; ++i) {
        const int h = order[i];
        if (h < 0 || h >= H || seen[h]) return SKSSM_ESHAPE;  // not a permutation
        seen[h] = 1;
        if (rank[h] > 0) sketch_seen = true;
        else if (sketch_seen) return SKSSM_ESHAPE;  // a dense head after a sketch head
    }
    return make_plan(shape, rank, group, order, out);
}

extern "C" sketchssm_status sketchssm_plan_export(const sketchssm_plan* p, int32_t* frame_index,
                                                  int32_t* frame_row_off, int32_t* z_row_off,
                                                  int32_t* bucket, int32_t* order,
                                                  int32_t* frame_group, int32_t* frame_rank,
                                                  int32_t* n_frames) {
    if (!p) return SKSSM_EINVAL;
    auto cp = [](int32_t* dst, const std::vector<int32_t>& src) {
        if (dst && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(int32_t));
    };
    cp(frame_index, p->frame_index);
    cp(frame_row_off, p->frame_row_off);
    cp(z_row_off, p->z_row_off);
    cp(bucket, p->bucket);
    cp(order, p->order);
    cp(frame_group, p->frame_group);
    cp(frame_rank, p->frame_rank);
    if (n_frames) *n_frames = p->n_frames;
    return SKSSM_OK;
}

extern "C" void sketchssm_plan_destroy(sketchssm_plan* p) { delete p; }

extern "C" size_t sketchssm_z_elems(const sketchssm_plan* p) { return p ? p->z_elems : 0; }

extern "C" size_t sketchssm_frame_elems(const sketchssm_plan* p) { return p ? p->frame_elems : 0; }

extern "C" const char* sketchssm_status_string(sketchssm_status s) {
    switch (s) {
        case SKSSM_OK: return "ok";
        case SKSSM_EINVAL: return "invalid argument (null pointer, enum, pos or n_tokens out of range)";
        case SKSSM_ESHAPE: return "unsupported shape or rank table";
        case SKSSM_EALIGN: return "device pointer not 16-byte aligned";
        case SKSSM_ENOMEM: return "host allocation failed";
        case SKSSM_EDEVICE: return "HIP runtime error";
        case SKSSM_ELAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}
