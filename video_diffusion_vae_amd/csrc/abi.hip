// Exported C entry points: argument validation, thread-local error reporting, the host-only tile
// split, and dispatch to the kernel launchers. No exception crosses this boundary.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "host.h"

namespace vae {

ErrorState& error_state() {
    static thread_local ErrorState st;
    return st;
}

vae_status_t fail(vae_status_t st, const std::string& msg, int32_t axis, int64_t extent,
                  int64_t multiple, int64_t min_width) {
    ErrorState& e = error_state();
    e.text = msg;
    e.info = vae_error_info_t{st, axis, extent, multiple, min_width};
    return st;
}

void clear_error() {
    ErrorState& e = error_state();
    e.text.clear();
    e.info = vae_error_info_t{VAE_OK, -1, -1, -1, -1};
}

// ------------------------------------------------------------------------------------------------
// Validation helpers
// ------------------------------------------------------------------------------------------------
vae_status_t check_tensor(const vae_tensor_t* t, const char* name) {
    if (!t) return fail(VAE_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (t->dtype != VAE_DTYPE_BF16 && t->dtype != VAE_DTYPE_F32 && t->dtype != VAE_DTYPE_F16)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": unknown dtype");
    const int64_t d[5] = {t->n, t->t, t->h, t->w, t->c};
    for (int i = 0; i < 5; ++i)
        if (d[i] < 0 || d[i] > INT32_MAX)
            return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": extent out of range", i, d[i]);
    if (t->c < 1) return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": no channels", 4, t->c);
    if (t->h * t->w > INT32_MAX || t->t * t->h > INT32_MAX)
        return fail(VAE_ERR_UNSUPPORTED, std::string(name) + ": spatial extent too large");
    if (numel(*t) > 0 && !t->data)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": data is NULL");
    if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": data must be 16-byte aligned");
    return VAE_OK;
}

vae_status_t check_box(const vae_box_t* b, const vae_tensor_t& t, const char* name) {
    if (!b) return VAE_OK;
    if (b->t0 < 0 || b->t0 > b->t1 || b->t1 > t.t)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": T range outside the tensor", 1, t.t);
    if (b->h0 < 0 || b->h0 > b->h1 || b->h1 > t.h)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": H range outside the tensor", 2, t.h);
    if (b->w0 < 0 || b->w0 > b->w1 || b->w1 > t.w)
        return fail(VAE_ERR_INVALID_ARG, std::string(name) + ": W range outside the tensor", 3, t.w);
    return VAE_OK;
}

bool overlaps(const vae_tensor_t& a, const vae_tensor_t& b) {
    const uint8_t* pa = static_cast<const uint8_t*>(a.data);
    const uint8_t* pb = static_cast<const uint8_t*>(b.data);
    const int64_t la = numel(a) * elem_size(a.dtype), lb = numel(b) * elem_size(b.dtype);
    if (la == 0 || lb == 0) return false;
    return pa < pb + lb && pb < pa + la;
}

bool same_grid(const vae_tensor_t& a, const vae_tensor_t& b) {
    return a.n == b.n && a.t == b.t && a.h == b.h && a.w == b.w;
}

vae_status_t box_list(const vae_tensor_t& x, const vae_box_t* boxes, int32_t n_boxes,
                      BoxList* out) {
    if (n_boxes < 1 || n_boxes > kMaxBoxes)
        return fail(VAE_ERR_UNSUPPORTED, "n_boxes must be in 1..16", -1, n_boxes, -1, 1);
    if (!boxes && n_boxes != 1) return fail(VAE_ERR_INVALID_ARG, "boxes is NULL but n_boxes > 1");
    out->n = n_boxes;
    for (int i = 0; i < n_boxes; ++i) {
        if (boxes) VAE_TRY(check_box(&boxes[i], x, "boxes[i]"));
        out->b[i] = to_box(boxes ? &boxes[i] : nullptr, x);
    }
    for (int i = 0; i < n_boxes; ++i)
        for (int j = 0; j < i; ++j) {
            const Box& a = out->b[i];
            const Box& b = out->b[j];
            if (a.volume() && b.volume() && a.t0 < b.t1 && b.t0 < a.t1 && a.h0 < b.h1 &&
                b.h0 < a.h1 && a.w0 < b.w1 && b.w0 < a.w1)
                return fail(VAE_ERR_INVALID_ARG, "boxes must not overlap");
        }
    return VAE_OK;
}

vae_status_t check_gn(const vae_tensor_t* x, int32_t groups) {
    VAE_TRY(check_tensor(x, "x"));
    if (groups < 1 || x->c % groups != 0)
        return fail(VAE_ERR_UNSUPPORTED, "channels must be divisible by groups", 4, x->c, groups);
    if (!gn_shape_supported(*x, groups))
        return fail(VAE_ERR_UNSUPPORTED,
                    "group norm needs C/vec to divide 256 and groups aligned to 16-byte vectors",
                    4, x->c, elem_size(x->dtype) == 2 ? 8 : 4);
    return VAE_OK;
}

// y: same shape as x; any dtype. In place only with the same dtype, otherwise disjoint.
vae_status_t check_gn_output(const vae_tensor_t& x, const vae_tensor_t& y) {
    if (!same_grid(x, y) || x.c != y.c)
        return fail(VAE_ERR_INVALID_ARG, "y must match x in shape");
    if (x.data == y.data && x.dtype == y.dtype) return VAE_OK;
    if (overlaps(x, y))
        return fail(VAE_ERR_INVALID_ARG, "y must be x itself (same dtype) or not overlap it");
    return VAE_OK;
}

size_t gn_full_workspace(const vae_tensor_t& x, const BoxList& bl, int32_t groups) {
    return align_up(gn_stats_workspace(x, bl, groups), 256) +
           align_up((size_t)x.n * groups * 2 * sizeof(float), 256);
}

// ------------------------------------------------------------------------------------------------
// Tile split (host integer maths)
// ------------------------------------------------------------------------------------------------
struct Band {
    int32_t start, size;
};

vae_status_t bands(int32_t length, int32_t parts, int axis, std::vector<Band>* out) {
    if (parts < 1)
        return fail(VAE_ERR_INVALID_ARG, "patch count must be >= 1", axis, parts, -1, 1);
    if (parts > length)
        // every patch needs at least one row: the one-row halo must come from a direct neighbour
        return fail(VAE_ERR_UNSUPPORTED, "a patch would be narrower than the one-row halo", axis,
                    length, -1, parts);
    const int32_t q = length / parts, r = length % parts;
    int32_t s = 0;
    out->clear();
    for (int32_t i = 0; i < parts; ++i) {
        const int32_t sz = i < r ? q + 1 : q;
        out->push_back(Band{s, sz});
        s += sz;
    }
    return VAE_OK;
}

vae_status_t check_tiling(const vae_tiling_desc_t* d) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "tiling desc is NULL");
    if (d->n < 1 || d->t < 1 || d->h < 1 || d->w < 1)
        return fail(VAE_ERR_INVALID_ARG, "latent extents must be >= 1");
    if (d->scale_t < 1 || d->scale_h < 1 || d->scale_w < 1)
        return fail(VAE_ERR_INVALID_ARG, "scales must be >= 1");
    if (d->down_t < 0 || d->down_h < 0 || d->down_w < 0)
        return fail(VAE_ERR_INVALID_ARG, "folds must be >= 0");
    if (encodes(*d)) {
        if (d->scale_t != 1 || d->scale_h != 1 || d->scale_w != 1 || d->tile_t > 0)
            return fail(VAE_ERR_UNSUPPORTED,
                        "an encoder tiling takes scales 1 and keeps T whole (tile_t = 0)");
        const int32_t ft = d->down_t > 1 ? d->down_t : 1, fh = d->down_h > 1 ? d->down_h : 1,
                      fw = d->down_w > 1 ? d->down_w : 1;
        if ((d->t + ft - 1) % ft)
            return fail(VAE_ERR_UNSUPPORTED, "T + down_t - 1 must be a multiple of down_t", 1,
                        d->t, ft);
        if (d->h % fh) return fail(VAE_ERR_UNSUPPORTED, "H must be a multiple of down_h", 2, d->h, fh);
        if (d->w % fw) return fail(VAE_ERR_UNSUPPORTED, "W must be a multiple of down_w", 3, d->w, fw);
    }
    if (d->mode == VAE_TILING_PATCH_HALO) {
        // an encoder's bands are whole multiples of its folds (P4, encoder commit)
        std::vector<Band> b;
        VAE_TRY(bands(d->h / std::max(d->down_h, 1), d->patches_h, 2, &b));
        VAE_TRY(bands(d->w / std::max(d->down_w, 1), d->patches_w, 3, &b));
    } else if (d->mode == VAE_TILING_OVERLAP_BLEND) {
        AxisTiling ax[3];
        overlap_axes(*d, ax);
        for (int i = 0; i < 3; ++i) {
            if (axis_is_cut(ax[i]) && (ax[i].stride < 1 || ax[i].stride > ax[i].tile))
                return fail(VAE_ERR_UNSUPPORTED, "tile stride must be in 1..tile (no gaps)",
                            1 + i, ax[i].stride, -1, 1);
        }
        if (axis_is_cut(ax[0]) && ax[0].scale > 1 && ax[0].stride >= ax[0].tile)
            return fail(VAE_ERR_UNSUPPORTED,
                        "temporal tiles must share a latent frame (stride_t < tile_t): a causal "
                        "tile's first frame would leave a gap",
                        1, ax[0].stride, -1, 1);
    } else {
        return fail(VAE_ERR_INVALID_ARG, "unknown tiling mode");
    }
    return VAE_OK;
}

int32_t out_frames(int32_t t, int32_t scale_t) { return 1 + (t - 1) * scale_t; }

vae_status_t check_fold(const vae_tensor_t& x, int32_t st, int32_t sh, int32_t sw) {
    if (st < 1 || sh < 1 || sw < 1) return fail(VAE_ERR_INVALID_ARG, "fold factors must be >= 1");
    if ((x.t + st - 1) % st)
        return fail(VAE_ERR_UNSUPPORTED, "s2d: T + st - 1 must be a multiple of st", 1, x.t, st);
    if (x.h % sh) return fail(VAE_ERR_UNSUPPORTED, "s2d: H must be a multiple of sh", 2, x.h, sh);
    if (x.w % sw) return fail(VAE_ERR_UNSUPPORTED, "s2d: W must be a multiple of sw", 3, x.w, sw);
    return VAE_OK;
}

bool encodes(const vae_tiling_desc_t& d) {
    return d.down_t > 1 || d.down_h > 1 || d.down_w > 1;
}

void desc_out_extents(const vae_tiling_desc_t& d, int32_t* t, int32_t* h, int32_t* w) {
    if (encodes(d)) {
        const int32_t ft = d.down_t > 1 ? d.down_t : 1;
        *t = (d.t + ft - 1) / ft;
        *h = d.h / (d.down_h > 1 ? d.down_h : 1);
        *w = d.w / (d.down_w > 1 ? d.down_w : 1);
        return;
    }
    *t = out_frames(d.t, d.scale_t);
    *h = d.h * d.scale_h;
    *w = d.w * d.scale_w;
}

void overlap_axes(const vae_tiling_desc_t& d, AxisTiling ax[3]) {
    if (encodes(d)) {   // cut on the output latent grid; T whole
        int32_t t, h, w;
        desc_out_extents(d, &t, &h, &w);
        ax[0] = AxisTiling{t, 0, 0, 1, 1};
        ax[1] = AxisTiling{h, d.tile_h, d.stride_h, 1, 0};
        ax[2] = AxisTiling{w, d.tile_w, d.stride_w, 1, 0};
        return;
    }
    ax[0] = AxisTiling{d.t, d.tile_t, d.stride_t, d.scale_t, 1};
    ax[1] = AxisTiling{d.h, d.tile_h, d.stride_h, d.scale_h, 0};
    ax[2] = AxisTiling{d.w, d.tile_w, d.stride_w, d.scale_w, 0};
}

std::vector<vae_tile_t> make_tiles(const vae_tiling_desc_t& d) {
    std::vector<vae_tile_t> tiles;
    const int32_t to = out_frames(d.t, d.scale_t);
    if (d.mode == VAE_TILING_PATCH_HALO && encodes(d)) {
        // bands in units of the fold: `latent` is the input-video box, `out` the latent box
        const int32_t fh = std::max(d.down_h, 1), fw = std::max(d.down_w, 1);
        int32_t ot, oh, ow;
        desc_out_extents(d, &ot, &oh, &ow);
        std::vector<Band> hb, wb;
        bands(oh, d.patches_h, 2, &hb);
        bands(ow, d.patches_w, 3, &wb);
        for (size_t i = 0; i < hb.size(); ++i)
            for (size_t j = 0; j < wb.size(); ++j) {
                vae_tile_t t{};
                t.index = (int32_t)tiles.size();
                t.row = (int32_t)i;
                t.col = (int32_t)j;
                t.latent = vae_box_t{0, d.t, hb[i].start * fh, (hb[i].start + hb[i].size) * fh,
                                     wb[j].start * fw, (wb[j].start + wb[j].size) * fw};
                t.out = vae_box_t{0, ot, hb[i].start, hb[i].start + hb[i].size, wb[j].start,
                                  wb[j].start + wb[j].size};
                tiles.push_back(t);
            }
    } else if (d.mode == VAE_TILING_PATCH_HALO) {
        std::vector<Band> hb, wb;
        bands(d.h, d.patches_h, 2, &hb);
        bands(d.w, d.patches_w, 3, &wb);
        for (size_t i = 0; i < hb.size(); ++i)
            for (size_t j = 0; j < wb.size(); ++j) {
                vae_tile_t t{};
                t.index = (int32_t)tiles.size();
                t.row = (int32_t)i;
                t.col = (int32_t)j;
                t.latent = vae_box_t{0, d.t, hb[i].start, hb[i].start + hb[i].size, wb[j].start,
                                     wb[j].start + wb[j].size};
                t.out = vae_box_t{0, to, hb[i].start * d.scale_h,
                                  (hb[i].start + hb[i].size) * d.scale_h, wb[j].start * d.scale_w,
                                  (wb[j].start + wb[j].size) * d.scale_w};
                tiles.push_back(t);
            }
    } else {
        AxisTiling ax[3];
        overlap_axes(d, ax);
        const AxisTiling &at = ax[0], &ah = ax[1], &aw = ax[2];
        for (int32_t k = 0; k < axis_count(at); ++k)
            for (int32_t i = 0; i < axis_count(ah); ++i)
                for (int32_t j = 0; j < axis_count(aw); ++j) {
                    int32_t ts, tn, hs, hn, ws, wn, ot, otn, oh, ohn, ow, own;
                    axis_span(at, k, &ts, &tn);
                    axis_span(ah, i, &hs, &hn);
                    axis_span(aw, j, &ws, &wn);
                    axis_out_span(at, k, &ot, &otn);
                    axis_out_span(ah, i, &oh, &ohn);
                    axis_out_span(aw, j, &ow, &own);
                    vae_tile_t t{};
                    t.index = (int32_t)tiles.size();
                    t.row = i;
                    t.col = j;
                    t.latent = vae_box_t{ts, ts + tn, hs, hs + hn, ws, ws + wn};
                    t.out = vae_box_t{ot, ot + otn, oh, oh + ohn, ow, ow + own};
                    if (encodes(d)) {   // the input-video box of the latent tile
                        const int32_t fh = d.down_h > 1 ? d.down_h : 1;
                        const int32_t fw = d.down_w > 1 ? d.down_w : 1;
                        t.latent = vae_box_t{0, d.t, hs * fh, (hs + hn) * fh, ws * fw,
                                             (ws + wn) * fw};
                    }
                    t.lead_t = axis_lead(at, k);
                    t.trail_t = axis_trail(at, k);
                    t.lead_h = axis_lead(ah, i);
                    t.trail_h = axis_trail(ah, i);
                    t.lead_w = axis_lead(aw, j);
                    t.trail_w = axis_trail(aw, j);
                    tiles.push_back(t);
                }
    }
    return tiles;
}

// The residual has y's shape, and y's dtype or fp32 when y is bf16 or fp16.
vae_status_t check_residual(const vae_tensor_t* r, const vae_tensor_t& x, const vae_tensor_t& y) {
    VAE_TRY(check_tensor(r, "residual"));
    const bool dtype_ok =
        r->dtype == y.dtype || (r->dtype == VAE_DTYPE_F32 && y.dtype != VAE_DTYPE_F32);
    if (!same_grid(*r, y) || r->c != y.c || !dtype_ok)
        return fail(VAE_ERR_INVALID_ARG,
                    "residual must match y in shape, and in dtype or be fp32 (bf16/fp16 y)");
    if (overlaps(*r, x)) return fail(VAE_ERR_INVALID_ARG, "residual overlaps x");
    return VAE_OK;
}

// fp16 tensors and the packed-weight flags (shared by both conv calls).
// `norm`: the conv normalises x while staging it (fp32 x with either packed flag, fp16 x with
// bf16-packed weights).
vae_status_t check_conv_dtypes(const vae_tensor_t& x, const vae_tensor_t& y,
                               const vae_tensor_t* residual, int64_t cout, int32_t weight_dtype,
                               int32_t flags, bool norm = false) {
    const int32_t packs = VAE_CONV_PACKED_WEIGHTS | VAE_CONV_PACKED_F16_WEIGHTS;
    if (flags & ~(VAE_CONV_SPLIT_FP32 | packs | VAE_CONV_SPLIT_K))
        return fail(VAE_ERR_INVALID_ARG, "unknown conv flags");
    if ((flags & packs) == packs)
        return fail(VAE_ERR_INVALID_ARG, "give one packed-weight flag");
    const bool mfma = conv_uses_mfma_c(x, cout, weight_dtype);
    if (x.dtype == VAE_DTYPE_F16 || y.dtype == VAE_DTYPE_F16) {
        if (!mfma)
            return fail(VAE_ERR_UNSUPPORTED,
                        "fp16 tensors need bf16 weights, Cin % 32 == 0 and Cout % 4 == 0", 4, x.c,
                        32);
        if (y.dtype == VAE_DTYPE_F16 && x.dtype == VAE_DTYPE_F32)
            return fail(VAE_ERR_UNSUPPORTED, "an fp16 y needs a bf16 or fp16 x");
    }
    if (norm) {
        if (!(flags & packs) || (flags & VAE_CONV_SPLIT_FP32) || !mfma)
            return fail(VAE_ERR_UNSUPPORTED,
                        "an input GroupNorm needs packed weights, no fp32 split, bf16 weights, "
                        "Cin % 32 == 0 and Cout % 4 == 0", 4, x.c, 32);
        if (x.dtype != VAE_DTYPE_F32 &&
            !(x.dtype == VAE_DTYPE_F16 && (flags & VAE_CONV_PACKED_WEIGHTS)))
            return fail(VAE_ERR_UNSUPPORTED, "an input GroupNorm reads fp32 x, or fp16 x with "
                                             "bf16-packed weights");
    } else {
        if ((flags & VAE_CONV_PACKED_F16_WEIGHTS) && x.dtype != VAE_DTYPE_F16)
            return fail(VAE_ERR_INVALID_ARG, "fp16-packed weights go with an fp16 x");
        if ((flags & VAE_CONV_PACKED_WEIGHTS) && x.dtype == VAE_DTYPE_F16)
            return fail(VAE_ERR_INVALID_ARG, "an fp16 x takes fp16-packed weights");
    }
    if ((flags & packs) && !mfma)
        return fail(VAE_ERR_UNSUPPORTED,
                    "packed weights need bf16 weights, Cin % 32 == 0 and Cout % 4 == 0", 4, x.c,
                    32);
    if (residual && residual->dtype != y.dtype && !mfma)
        return fail(VAE_ERR_UNSUPPORTED, "an fp32 residual with a bf16 y needs the MFMA path");
    return VAE_OK;
}

vae_status_t check_conv(const vae_tensor_t* x, const void* weight, int32_t weight_dtype,
                        const vae_tensor_t* residual, vae_tensor_t* y, const vae_box_t* out_box,
                        int32_t flags) {
    VAE_TRY(check_tensor(x, "x"));
    VAE_TRY(check_tensor(y, "y"));
    if (!weight) return fail(VAE_ERR_INVALID_ARG, "weight is NULL");
    if (weight_dtype != VAE_DTYPE_BF16 && weight_dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_INVALID_ARG, "unknown weight dtype");
    if (reinterpret_cast<uintptr_t>(weight) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "weight must be 16-byte aligned");
    if (!same_grid(*x, *y)) return fail(VAE_ERR_INVALID_ARG, "x and y must share N, T, H, W");
    if (residual) VAE_TRY(check_residual(residual, *x, *y));
    if (overlaps(*x, *y)) return fail(VAE_ERR_INVALID_ARG, "y must not overlap x");
    VAE_TRY(check_box(out_box, *y, "out_box"));
    if (flags & VAE_CONV_SPLIT_K)
        return fail(VAE_ERR_INVALID_ARG,
                    "VAE_CONV_SPLIT_K needs a workspace: use vae_conv3d_causal_fused");
    VAE_TRY(check_conv_dtypes(*x, *y, residual, y->c, weight_dtype, flags));
    return VAE_OK;
}

// The fused call's depth-to-space factors (0, 0, 0 reads as 1, 1, 1) and the box of y that the
// conv's out_box covers.
struct FusedPlan {
    int32_t st, sh, sw, k;
    int32_t lsh, lsw;     // log2 of the input's nearest upsampling (0 = none)
    Box cbox, ybox;
};

// log2 of a nearest factor: 0 reads as 1; factors must be powers of two up to 16.
int32_t nearest_log2(int32_t f) {
    if (f == 0 || f == 1) return 0;
    for (int32_t l = 1; l <= 4; ++l)
        if (f == (1 << l)) return l;
    return -1;
}

// `run`: the call itself (the workspace query needs no output pointers).
vae_status_t check_fused(const vae_conv_fused_t* a, FusedPlan* p, bool run) {
    if (!a) return fail(VAE_ERR_INVALID_ARG, "args is NULL");
    VAE_TRY(check_tensor(a->x, "x"));
    VAE_TRY(check_tensor(a->y, "y"));
    const vae_tensor_t& x = *a->x;
    const vae_tensor_t& y = *a->y;
    if (!a->weight) return fail(VAE_ERR_INVALID_ARG, "weight is NULL");
    if (a->weight_dtype != VAE_DTYPE_BF16 && a->weight_dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_INVALID_ARG, "unknown weight dtype");
    p->lsh = nearest_log2(a->in_up_sh);
    p->lsw = nearest_log2(a->in_up_sw);
    if (p->lsh < 0 || p->lsw < 0)
        return fail(VAE_ERR_UNSUPPORTED, "input upsampling factors must be 0, 1, 2, 4, 8 or 16");
    // the conv's input grid: x after the nearest upsampling
    vae_tensor_t xl = x;
    xl.h = x.h << p->lsh;
    xl.w = x.w << p->lsw;
    if (xl.h * xl.w > INT32_MAX)
        return fail(VAE_ERR_UNSUPPORTED, "upsampled spatial extent too large");
    if (reinterpret_cast<uintptr_t>(a->weight) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "weight must be 16-byte aligned");
    const bool none = a->d2s_st == 0 && a->d2s_sh == 0 && a->d2s_sw == 0;
    p->st = none ? 1 : a->d2s_st;
    p->sh = none ? 1 : a->d2s_sh;
    p->sw = none ? 1 : a->d2s_sw;
    if (p->st < 1 || p->sh < 1 || p->sw < 1)
        return fail(VAE_ERR_INVALID_ARG, "d2s factors must all be 0 or all be >= 1");
    p->k = p->st * p->sh * p->sw;
    if (y.n != xl.n || y.t != p->st * xl.t - (p->st - 1) || y.h != p->sh * xl.h ||
        y.w != p->sw * xl.w)
        return fail(VAE_ERR_INVALID_ARG,
                    "y must be [N, st*T-(st-1), sh*H, sw*W, Cout/(st*sh*sw)] of the input grid "
                    "[N, T, H, W] (x's, times the input upsampling)");
    if (a->residual) VAE_TRY(check_residual(a->residual, x, y));
    if (overlaps(x, y)) return fail(VAE_ERR_INVALID_ARG, "y must not overlap x");
    VAE_TRY(check_box(a->out_box, xl, "out_box"));
    p->cbox = to_box(a->out_box, xl);
    const Box& b = p->cbox;
    p->ybox = Box{std::max(0, p->st * b.t0 - (p->st - 1)), p->st * b.t1 - (p->st - 1),
                  p->sh * b.h0, p->sh * b.h1, p->sw * b.w0, p->sw * b.w1};
    const bool mfma = conv_uses_mfma_c(x, y.c * p->k, a->weight_dtype);
    const bool norm = a->in_scale_shift != nullptr;
    VAE_TRY(check_conv_dtypes(x, y, a->residual, y.c * p->k, a->weight_dtype, a->flags, norm));
    if (norm && reinterpret_cast<uintptr_t>(a->in_scale_shift) % 16)
        return fail(VAE_ERR_INVALID_ARG, "in_scale_shift must be 16-byte aligned");
    if ((p->k > 1 || p->lsh || p->lsw) && !mfma)
        return fail(VAE_ERR_UNSUPPORTED,
                    "a fused depth-to-space or input upsampling needs bf16 weights, Cin % 32 == 0 "
                    "and Cout % 4 == 0", 4, x.c, 32);
    if (a->gn_groups) {
        if (y.dtype == VAE_DTYPE_F16)
            return fail(VAE_ERR_UNSUPPORTED, "statistics of an fp16 y are not gathered");
        VAE_TRY(check_gn(a->y, a->gn_groups));
        if (!(a->gn_eps >= 0.0f)) return fail(VAE_ERR_INVALID_ARG, "gn_eps must be >= 0");
        if (run && !a->gn_mean_rstd) return fail(VAE_ERR_INVALID_ARG, "gn_mean_rstd is NULL");
    }
    return VAE_OK;
}

// Workspace of the fused call: the epilogue's partials, or the separate statistics pass's; then,
// 256-byte aligned at `split_off`, the partial sums of a split over K (`splits` > 1).
size_t fused_workspace(const vae_conv_fused_t* a, const FusedPlan& p, int64_t* slots,
                       int32_t* splits, size_t* split_off) {
    *slots = 0;
    size_t gn = 0;
    if (a->gn_groups) {
        *slots = conv_gn_slots(*a->x, a->y->c, a->weight_dtype, p.cbox, a->gn_groups, p.k,
                               (a->flags & VAE_CONV_SPLIT_K) != 0);
        if (*slots > 0) {
            gn = (size_t)(a->y->n * a->gn_groups * *slots * 3) * sizeof(double);
        } else {
            BoxList bl;
            bl.n = 1;
            bl.b[0] = p.ybox;
            gn = gn_stats_workspace(*a->y, bl, a->gn_groups);
        }
    }
    vae_tensor_t xl = *a->x;                 // the conv's input grid
    xl.h <<= p.lsh;
    xl.w <<= p.lsw;
    const int64_t cout = a->y->c * p.k;
    *splits = (a->flags & VAE_CONV_SPLIT_K)
                  ? conv_split_count(xl, cout, a->weight_dtype, p.cbox,
                                     (a->flags & VAE_CONV_SPLIT_FP32) != 0)
                  : 1;
    *split_off = align_up(gn, 256);
    const size_t sb = conv_split_bytes(xl, cout, p.cbox, *splits);
    return sb ? *split_off + sb : gn;
}

vae_status_t check_attention(const vae_tensor_t* x) {
    VAE_TRY(check_tensor(x, "x"));
    if (x->dtype != VAE_DTYPE_F32) return fail(VAE_ERR_UNSUPPORTED, "attention reads fp32 x");
    if (!attention_shape_supported(x->c))
        return fail(VAE_ERR_UNSUPPORTED, "attention needs C % 32 == 0 and C / 8 dividing 256", 4,
                    x->c, 32);
    return VAE_OK;
}

}  // namespace vae

using namespace vae;

extern "C" {

VAE_API const char* vae_last_error(void) { return error_state().text.c_str(); }

VAE_API vae_status_t vae_last_error_info(vae_error_info_t* info) {
    if (!info) return VAE_ERR_INVALID_ARG;
    *info = error_state().info;
    return VAE_OK;
}

VAE_API int32_t vae_version(void) { return 100; }


VAE_API vae_status_t vae_conv3d_causal(const vae_tensor_t* x, const void* weight,
                                       int32_t weight_dtype, const float* bias,
                                       const vae_tensor_t* residual, vae_tensor_t* y,
                                       const vae_box_t* out_box, int32_t flags,
                                       vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_conv(x, weight, weight_dtype, residual, y, out_box, flags));
    return launch_conv3d(*x, weight, weight_dtype, bias, residual, *y, to_box(out_box, *y), flags,
                         as_stream(stream));
}

VAE_API vae_status_t vae_conv3d_causal_fused_workspace(const vae_conv_fused_t* args,
                                                       size_t* bytes) {
    clear_error();
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "bytes is NULL");
    FusedPlan p;
    VAE_TRY(check_fused(args, &p, false));
    int64_t slots = 0;
    int32_t splits = 1;
    size_t split_off = 0;
    *bytes = fused_workspace(args, p, &slots, &splits, &split_off);
    return VAE_OK;
}

VAE_API vae_status_t vae_conv3d_causal_fused(const vae_conv_fused_t* args, vae_stream_t stream) {
    clear_error();
    FusedPlan p;
    VAE_TRY(check_fused(args, &p, true));
    const vae_conv_fused_t& a = *args;
    const vae_tensor_t& x = *a.x;
    const vae_tensor_t& y = *a.y;
    int64_t slots = 0;
    int32_t splits = 1;
    size_t split_off = 0;
    const size_t need = fused_workspace(args, p, &slots, &splits, &split_off);
    if (a.gn_groups || splits > 1) {
        if (!a.ws || a.ws_bytes < need)
            return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)a.ws_bytes, -1,
                        (int64_t)need);
        if (reinterpret_cast<uintptr_t>(a.ws) % 16 != 0)
            return fail(VAE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    if (a.gn_groups && (p.cbox.volume() == 0 || p.ybox.volume() == 0 || x.n == 0))
        return fail(VAE_ERR_INVALID_ARG, "statistics of an empty box");
    hipStream_t s = as_stream(stream);
    double* part = static_cast<double*>(a.ws);
    ConvFuse fz{slots > 0 ? part : nullptr, a.gn_groups ? a.gn_groups : 1, p.st, p.sh, p.sw,
                p.lsh, p.lsw};
    if (splits > 1) {
        fz.part = reinterpret_cast<float*>(static_cast<uint8_t*>(a.ws) + split_off);
        fz.splits = splits;
    }
    fz.in_ab = a.in_scale_shift;
    VAE_TRY(launch_conv3d(x, a.weight, a.weight_dtype, a.bias, a.residual, y, p.cbox, a.flags, s,
                          &fz));
    if (!a.gn_groups) return VAE_OK;
    if (slots > 0)
        return launch_gn_finalize_slots(part, slots, (int32_t)y.n, a.gn_groups, a.gn_eps,
                                        a.gn_mean_rstd, s);
    BoxList bl;
    bl.n = 1;
    bl.b[0] = p.ybox;
    return launch_gn_stats(y, bl, a.gn_groups, part, nullptr, a.gn_mean_rstd, a.gn_eps, s);
}

VAE_API vae_status_t vae_conv3d_causal_strided(const vae_tensor_t* x, const void* weight,
                                               int32_t weight_dtype, const float* bias,
                                               const vae_tensor_t* residual, vae_tensor_t* y,
                                               const vae_box_t* out_box, int32_t st, int32_t sh,
                                               int32_t sw, int32_t pad, int32_t flags,
                                               vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_tensor(x, "x"));
    VAE_TRY(check_tensor(y, "y"));
    if (!weight) return fail(VAE_ERR_INVALID_ARG, "weight is NULL");
    if (weight_dtype != VAE_DTYPE_BF16 && weight_dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_INVALID_ARG, "unknown weight dtype");
    if (reinterpret_cast<uintptr_t>(weight) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "weight must be 16-byte aligned");
    if (st < 1 || sh < 1 || sw < 1) return fail(VAE_ERR_INVALID_ARG, "strides must be >= 1");
    if (pad != VAE_PAD_AROUND && pad != VAE_PAD_AFTER)
        return fail(VAE_ERR_INVALID_ARG, "pad must be VAE_PAD_AROUND or VAE_PAD_AFTER");
    const int32_t packs = VAE_CONV_PACKED_WEIGHTS | VAE_CONV_PACKED_F16_WEIGHTS;
    if (flags & ~packs) return fail(VAE_ERR_INVALID_ARG, "unknown flags for a strided conv");
    if ((flags & packs) == packs) return fail(VAE_ERR_INVALID_ARG, "give one packed-weight flag");
    const int32_t before = pad == VAE_PAD_AROUND ? 1 : 0;
    const int64_t ot = (x->t - 1) / st + 1;
    const int64_t oh = (x->h + before + 1 - 3) / sh + 1;
    const int64_t ow = (x->w + before + 1 - 3) / sw + 1;
    if (x->h + before + 1 < 3 || x->w + before + 1 < 3)
        return fail(VAE_ERR_INVALID_ARG, "strided conv: the padded image is narrower than 3");
    if (y->n != x->n || y->t != ot || y->h != oh || y->w != ow)
        return fail(VAE_ERR_INVALID_ARG,
                    "y must be [N, (T-1)/st+1, (H+pt+pb-3)/sh+1, (W+pl+pr-3)/sw+1, Cout]");
    if (residual) {
        VAE_TRY(check_tensor(residual, "residual"));
        if (residual->n != y->n || residual->t != y->t || residual->h != y->h ||
            residual->w != y->w || residual->c != y->c ||
            (residual->dtype != y->dtype && residual->dtype != VAE_DTYPE_F32))
            return fail(VAE_ERR_INVALID_ARG, "residual must have y's shape, y's dtype or fp32");
        if (overlaps(*residual, *x)) return fail(VAE_ERR_INVALID_ARG, "residual overlaps x");
    }
    if (overlaps(*x, *y)) return fail(VAE_ERR_INVALID_ARG, "y must not overlap x");
    VAE_TRY(check_box(out_box, *y, "out_box"));
    const StrideGeom g{st, sh, sw, before, before};
    const bool mfma = conv_strided_uses_mfma(*x, y->c, weight_dtype, flags, g);
    if ((flags & packs) && !mfma)
        return fail(VAE_ERR_UNSUPPORTED,
                    "strided conv: packed weights need a bf16 or fp16 x, Cin % 32 == 0, "
                    "Cout % 4 == 0, st and sh = sw in {1, 2}", 4, x->c, 32);
    if (!mfma && (x->dtype == VAE_DTYPE_F16 || y->dtype == VAE_DTYPE_F16))
        return fail(VAE_ERR_UNSUPPORTED, "strided conv: fp16 tensors need packed weights");
    if (residual && residual->dtype != y->dtype && !mfma)
        return fail(VAE_ERR_UNSUPPORTED, "strided conv: an fp32 residual with a 2-byte y needs "
                                         "the matrix-core path");
    return launch_conv3d_strided(*x, weight, weight_dtype, bias, residual, *y, to_box(out_box, *y),
                                 g, flags, as_stream(stream));
}

VAE_API vae_status_t vae_conv_weight_pack_size(int32_t cout, int32_t cin, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "bytes is NULL");
    if (cout < 1 || cin < 1) return fail(VAE_ERR_INVALID_ARG, "cout and cin must be >= 1");
    if (cin % 32) return fail(VAE_ERR_UNSUPPORTED, "packing needs Cin % 32 == 0", 4, cin, 32);
    *bytes = (size_t)packed_weight_elems(cout, cin) * 2;
    return VAE_OK;
}

VAE_API vae_status_t vae_conv_weight_pack(const void* weight, int32_t cout, int32_t cin,
                                          void* packed, vae_stream_t stream) {
    clear_error();
    if (!weight || !packed) return fail(VAE_ERR_INVALID_ARG, "weight or packed is NULL");
    if (cout < 1 || cin < 1) return fail(VAE_ERR_INVALID_ARG, "cout and cin must be >= 1");
    if (cin % 32) return fail(VAE_ERR_UNSUPPORTED, "packing needs Cin % 32 == 0", 4, cin, 32);
    if (reinterpret_cast<uintptr_t>(packed) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "packed must be 16-byte aligned");
    return launch_pack_weights(weight, cout, cin, packed, as_stream(stream));
}

VAE_API vae_status_t vae_conv_weight_pack_f16(const void* weight, int32_t cout, int32_t cin,
                                              void* packed, vae_stream_t stream) {
    clear_error();
    if (!weight || !packed) return fail(VAE_ERR_INVALID_ARG, "weight or packed is NULL");
    if (cout < 1 || cin < 1) return fail(VAE_ERR_INVALID_ARG, "cout and cin must be >= 1");
    if (cin % 32) return fail(VAE_ERR_UNSUPPORTED, "packing needs Cin % 32 == 0", 4, cin, 32);
    if (reinterpret_cast<uintptr_t>(packed) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "packed must be 16-byte aligned");
    return launch_pack_weights(weight, cout, cin, packed, as_stream(stream), true);
}

VAE_API vae_status_t vae_groupnorm_stats_workspace(const vae_tensor_t* x, const vae_box_t* boxes,
                                                   int32_t n_boxes, int32_t groups,
                                                   size_t* bytes) {
    clear_error();
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "bytes is NULL");
    VAE_TRY(check_gn(x, groups));
    BoxList bl;
    VAE_TRY(box_list(*x, boxes, n_boxes, &bl));
    *bytes = gn_stats_workspace(*x, bl, groups);
    return VAE_OK;
}

VAE_API vae_status_t vae_groupnorm_silu_workspace(const vae_tensor_t* x, const vae_box_t* boxes,
                                                  int32_t n_boxes, int32_t groups, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "bytes is NULL");
    VAE_TRY(check_gn(x, groups));
    BoxList bl;
    VAE_TRY(box_list(*x, boxes, n_boxes, &bl));
    *bytes = gn_full_workspace(*x, bl, groups);
    return VAE_OK;
}

VAE_API vae_status_t vae_groupnorm_stats(const vae_tensor_t* x, const vae_box_t* boxes,
                                         int32_t n_boxes, int32_t groups, double* part, void* ws,
                                         size_t ws_bytes, vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_gn(x, groups));
    BoxList bl;
    VAE_TRY(box_list(*x, boxes, n_boxes, &bl));
    if (!part) return fail(VAE_ERR_INVALID_ARG, "part is NULL");
    const size_t need = gn_stats_workspace(*x, bl, groups);
    if (!ws || ws_bytes < need)
        return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)ws_bytes, -1,
                    (int64_t)need);
    return launch_gn_stats(*x, bl, groups, static_cast<double*>(ws), part, nullptr, 0.0f,
                           as_stream(stream));
}

VAE_API vae_status_t vae_groupnorm_combine(const double* part, int32_t n_parts, int32_t n,
                                           int32_t groups, float eps, float* mean_rstd,
                                           vae_stream_t stream) {
    clear_error();
    if (!part || !mean_rstd) return fail(VAE_ERR_INVALID_ARG, "part or mean_rstd is NULL");
    if (n_parts < 1 || n < 1 || groups < 1 || !(eps >= 0.0f))
        return fail(VAE_ERR_INVALID_ARG, "n_parts, n, groups must be >= 1 and eps >= 0");
    return launch_gn_combine(part, n_parts, n, groups, eps, mean_rstd, as_stream(stream));
}

VAE_API vae_status_t vae_groupnorm_apply(const vae_tensor_t* x, const vae_box_t* box,
                                         int32_t groups, const float* mean_rstd,
                                         const float* gamma, const float* beta,
                                         int32_t apply_silu, vae_tensor_t* y,
                                         vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_gn(x, groups));
    VAE_TRY(check_tensor(y, "y"));
    VAE_TRY(check_gn_output(*x, *y));
    if (!mean_rstd) return fail(VAE_ERR_INVALID_ARG, "mean_rstd is NULL");
    VAE_TRY(check_box(box, *x, "box"));
    return launch_gn_apply(*x, to_box(box, *x), groups, mean_rstd, gamma, beta, apply_silu != 0,
                           *y, as_stream(stream));
}

VAE_API vae_status_t vae_groupnorm_scale_shift(const float* mean_rstd, int32_t n, int32_t channels,
                                               int32_t groups, const float* gamma,
                                               const float* beta, float* scale_shift,
                                               vae_stream_t stream) {
    clear_error();
    if (!mean_rstd || !scale_shift)
        return fail(VAE_ERR_INVALID_ARG, "mean_rstd and scale_shift must not be NULL");
    if (n < 0 || groups < 1 || channels < 1 || channels % groups || channels % 8)
        return fail(VAE_ERR_INVALID_ARG,
                    "need n >= 0, groups >= 1 and channels a multiple of groups and of 8", 4,
                    channels, 8);
    if (reinterpret_cast<uintptr_t>(scale_shift) % 16)
        return fail(VAE_ERR_INVALID_ARG, "scale_shift must be 16-byte aligned");
    return launch_gn_scale_shift(mean_rstd, n, channels, groups, gamma, beta, scale_shift,
                                 as_stream(stream));
}

VAE_API vae_status_t vae_groupnorm_silu(const vae_tensor_t* x, const vae_box_t* boxes,
                                        int32_t n_boxes, int32_t groups, float eps,
                                        const float* gamma, const float* beta, int32_t apply_silu,
                                        vae_tensor_t* y, void* ws, size_t ws_bytes,
                                        vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_gn(x, groups));
    VAE_TRY(check_tensor(y, "y"));
    VAE_TRY(check_gn_output(*x, *y));
    if (!(eps >= 0.0f)) return fail(VAE_ERR_INVALID_ARG, "eps must be >= 0");
    BoxList bl;
    VAE_TRY(box_list(*x, boxes, n_boxes, &bl));
    const size_t need = gn_full_workspace(*x, bl, groups);
    if (!ws || ws_bytes < need)
        return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)ws_bytes, -1,
                    (int64_t)need);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(VAE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    double* stats = static_cast<double*>(ws);
    float* mr = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                         align_up(gn_stats_workspace(*x, bl, groups), 256));
    hipStream_t s = as_stream(stream);
    VAE_TRY(launch_gn_stats(*x, bl, groups, stats, nullptr, mr, eps, s));
    for (int i = 0; i < bl.n; ++i)
        VAE_TRY(launch_gn_apply(*x, bl.b[i], groups, mr, gamma, beta, apply_silu != 0, *y, s));
    return VAE_OK;
}

}  // extern "C"

namespace vae {
namespace {

// Scratch of vae_groupnorm_silu_noalloc: one copy per GPU, held from the library's load until the
// process ends. In host code `gn_scratch` stands for the array, not its device address: kernels
// get the address hipGetSymbolAddress returns on that device.
constexpr size_t kGnScratchBytes = size_t(8) << 20;
__device__ __align__(256) uint8_t gn_scratch[kGnScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex gn_scratch_mutex;
uint8_t* gn_scratch_ptr[kMaxDevices];   // per device, null until its first call

// The current device's scratch address, looked up once per device (with that device current).
vae_status_t gn_scratch_address(uint8_t** out) {
    int dev = -1;
    VAE_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(VAE_ERR_UNSUPPORTED, "device index beyond the library's table");
    std::lock_guard<std::mutex> lock(gn_scratch_mutex);
    if (!gn_scratch_ptr[dev]) {
        void* p = nullptr;
        VAE_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(gn_scratch)));
        if (!p) return fail(VAE_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch");
        gn_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *out = gn_scratch_ptr[dev];
    return VAE_OK;
}

}  // namespace
}  // namespace vae

extern "C" {

VAE_API vae_status_t vae_groupnorm_silu_noalloc(const vae_tensor_t* x, const vae_box_t* boxes,
                                                int32_t n_boxes, int32_t groups, float eps,
                                                const float* gamma, const float* beta,
                                                int32_t apply_silu, vae_tensor_t* y,
                                                vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_gn(x, groups));
    VAE_TRY(check_tensor(y, "y"));
    VAE_TRY(check_gn_output(*x, *y));
    if (!(eps >= 0.0f)) return fail(VAE_ERR_INVALID_ARG, "eps must be >= 0");
    BoxList bl;
    VAE_TRY(box_list(*x, boxes, n_boxes, &bl));
    const size_t need = gn_full_workspace(*x, bl, groups);
    if (need > kGnScratchBytes)
        return fail(VAE_ERR_UNSUPPORTED,
                    "vae_groupnorm_silu_noalloc: this call needs " + std::to_string(need) +
                        " bytes of scratch, above the library's " +
                        std::to_string(kGnScratchBytes) + " (use vae_groupnorm_silu)",
                    -1, (int64_t)need, -1, (int64_t)kGnScratchBytes);
    uint8_t* ws = nullptr;
    VAE_TRY(gn_scratch_address(&ws));
    // the same launches as vae_groupnorm_silu: every partial slot the merge reads is written
    // first by the statistics pass, so nothing needs clearing between calls
    double* stats = reinterpret_cast<double*>(ws);
    float* mr = reinterpret_cast<float*>(ws + align_up(gn_stats_workspace(*x, bl, groups), 256));
    hipStream_t s = as_stream(stream);
    VAE_TRY(launch_gn_stats(*x, bl, groups, stats, nullptr, mr, eps, s));
    for (int i = 0; i < bl.n; ++i)
        VAE_TRY(launch_gn_apply(*x, bl.b[i], groups, mr, gamma, beta, apply_silu != 0, *y, s));
    return VAE_OK;
}

VAE_API vae_status_t vae_rmsnorm_silu(const vae_tensor_t* x, float eps, const float* gamma,
                                      const float* beta, int32_t apply_silu, vae_tensor_t* y,
                                      vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_tensor(x, "x"));
    VAE_TRY(check_tensor(y, "y"));
    if (!rms_shape_supported(x->c))
        return fail(VAE_ERR_UNSUPPORTED, "rms norm needs C % 8 == 0 and C / 8 dividing 256", 4,
                    x->c, 8);
    if (!(eps >= 0.0f)) return fail(VAE_ERR_INVALID_ARG, "eps must be >= 0");
    VAE_TRY(check_gn_output(*x, *y));
    return launch_rms_norm(*x, eps, gamma, beta, apply_silu != 0, *y, as_stream(stream));
}

VAE_API vae_status_t vae_frame_attention_workspace(const vae_tensor_t* x, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "bytes is NULL");
    VAE_TRY(check_attention(x));
    *bytes = attention_workspace(*x);
    return VAE_OK;
}

VAE_API vae_status_t vae_frame_attention(const vae_tensor_t* x, float eps, const float* gamma,
                                         const float* beta, const void* w_qkv,
                                         const float* b_qkv, const void* w_out,
                                         const float* b_out, vae_tensor_t* y, void* ws,
                                         size_t ws_bytes, vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_attention(x));
    VAE_TRY(check_tensor(y, "y"));
    if (y->dtype != VAE_DTYPE_F32 || !same_grid(*x, *y) || y->c != x->c)
        return fail(VAE_ERR_INVALID_ARG, "y must be fp32 with x's shape");
    if (y->data != x->data && overlaps(*x, *y))
        return fail(VAE_ERR_INVALID_ARG, "y must be x itself or not overlap it");
    if (!w_qkv || !w_out) return fail(VAE_ERR_INVALID_ARG, "w_qkv or w_out is NULL");
    if (reinterpret_cast<uintptr_t>(w_qkv) % 16 || reinterpret_cast<uintptr_t>(w_out) % 16)
        return fail(VAE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
    if (!(eps >= 0.0f)) return fail(VAE_ERR_INVALID_ARG, "eps must be >= 0");
    const size_t need = attention_workspace(*x);
    if (numel(*x) > 0 && (!ws || ws_bytes < need))
        return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)ws_bytes, -1,
                    (int64_t)need);
    if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return fail(VAE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return launch_frame_attention(*x, eps, gamma, beta, w_qkv, b_qkv, w_out, b_out, *y, ws,
                                  as_stream(stream));
}

VAE_API vae_status_t vae_upsample(const vae_tensor_t* x, const vae_box_t* box, int32_t mode,
                                  int32_t st, int32_t sh, int32_t sw, vae_tensor_t* y,
                                  vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_tensor(x, "x"));
    VAE_TRY(check_tensor(y, "y"));
    if (st < 1 || sh < 1 || sw < 1) return fail(VAE_ERR_INVALID_ARG, "factors must be >= 1");
    if (x->dtype != y->dtype) return fail(VAE_ERR_INVALID_ARG, "x and y dtypes differ");
    if (x->n != y->n) return fail(VAE_ERR_INVALID_ARG, "x and y batch differ");
    if (mode == VAE_UPSAMPLE_D2S) {
        const int64_t k = (int64_t)st * sh * sw;
        if (x->c != y->c * k)
            return fail(VAE_ERR_INVALID_ARG, "d2s: x channels must be y channels * st*sh*sw", 4,
                        x->c, k);
        if (y->t != st * x->t - (st - 1) || y->h != x->h * sh || y->w != x->w * sw)
            return fail(VAE_ERR_INVALID_ARG, "d2s: y shape must be (st*T-(st-1), sh*H, sw*W)");
    } else if (mode == VAE_UPSAMPLE_NEAREST) {
        if (st != 1) return fail(VAE_ERR_UNSUPPORTED, "nearest: temporal factor must be 1");
        if (x->c != y->c || y->t != x->t || y->h != x->h * sh || y->w != x->w * sw)
            return fail(VAE_ERR_INVALID_ARG, "nearest: y shape must be (T, sh*H, sw*W, C)");
    } else {
        return fail(VAE_ERR_INVALID_ARG, "unknown upsample mode");
    }
    if (overlaps(*x, *y)) return fail(VAE_ERR_INVALID_ARG, "y must not overlap x");
    VAE_TRY(check_box(box, *x, "box"));
    return launch_upsample(*x, to_box(box, *x), mode, st, sh, sw, *y, as_stream(stream));
}

VAE_API vae_status_t vae_space_to_depth(const vae_tensor_t* x, int32_t st, int32_t sh, int32_t sw,
                                        vae_tensor_t* y, vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_tensor(x, "x"));
    VAE_TRY(check_tensor(y, "y"));
    VAE_TRY(check_fold(*x, st, sh, sw));
    const int64_t k = (int64_t)st * sh * sw;
    if (x->dtype != y->dtype) return fail(VAE_ERR_INVALID_ARG, "x and y dtypes differ");
    if (y->n != x->n || y->t != (x->t + st - 1) / st || y->h != x->h / sh ||
        y->w != x->w / sw || y->c != x->c * k)
        return fail(VAE_ERR_INVALID_ARG,
                    "s2d: y shape must be ((T+st-1)/st, H/sh, W/sw, C*st*sh*sw)");
    if (overlaps(*x, *y)) return fail(VAE_ERR_INVALID_ARG, "y must not overlap x");
    return launch_space_to_depth(*x, st, sh, sw, *y, as_stream(stream));
}

VAE_API vae_status_t vae_tile_split(const vae_tiling_desc_t* desc, vae_tile_t* tiles,
                                    int32_t capacity, int32_t* n_tiles) {
    clear_error();
    if (!n_tiles) return fail(VAE_ERR_INVALID_ARG, "n_tiles is NULL");
    VAE_TRY(check_tiling(desc));
    std::vector<vae_tile_t> v;
    try {
        v = make_tiles(*desc);
    } catch (const std::bad_alloc&) {
        return fail(VAE_ERR_INVALID_ARG, "out of host memory");
    }
    *n_tiles = (int32_t)v.size();
    if (!tiles) return VAE_OK;
    if (capacity < (int32_t)v.size())
        return fail(VAE_ERR_INVALID_ARG, "capacity smaller than the tile count", -1, capacity, -1,
                    (int64_t)v.size());
    std::memcpy(tiles, v.data(), v.size() * sizeof(vae_tile_t));
    return VAE_OK;
}

VAE_API vae_status_t vae_tile_merge(const vae_tensor_t* tile_out, const vae_tile_t* tile,
                                    const vae_tiling_desc_t* desc, vae_tensor_t* out,
                                    int32_t flags, vae_stream_t stream) {
    clear_error();
    VAE_TRY(check_tensor(tile_out, "tile_out"));
    VAE_TRY(check_tensor(out, "out"));
    VAE_TRY(check_tiling(desc));
    if (!tile) return fail(VAE_ERR_INVALID_ARG, "tile is NULL");
    if (desc->mode != VAE_TILING_OVERLAP_BLEND)
        return fail(VAE_ERR_INVALID_ARG, "merge takes an overlap-blend tiling");
    if (tile_out->dtype != VAE_DTYPE_F32 || out->dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_UNSUPPORTED, "merge accumulates fp32 tensors");
    int32_t ot, oh, ow;
    desc_out_extents(*desc, &ot, &oh, &ow);
    if (out->n != desc->n || out->t != ot || out->h != oh || out->w != ow)
        return fail(VAE_ERR_INVALID_ARG, "out shape does not match the tiling");
    const vae_box_t& ob = tile->out;
    VAE_TRY(check_box(&ob, *out, "tile->out"));
    if (tile_out->n != out->n || tile_out->c != out->c || tile_out->t != ob.t1 - ob.t0 ||
        tile_out->h != ob.h1 - ob.h0 || tile_out->w != ob.w1 - ob.w0)
        return fail(VAE_ERR_INVALID_ARG, "tile_out shape must be the tile's output box");
    if (overlaps(*tile_out, *out)) return fail(VAE_ERR_INVALID_ARG, "tile_out overlaps out");
    if (flags & ~(VAE_MERGE_ZERO | VAE_MERGE_FINALIZE))
        return fail(VAE_ERR_INVALID_ARG, "unknown merge flags");
    hipStream_t s = as_stream(stream);
    if (flags & VAE_MERGE_ZERO) VAE_TRY(launch_zero(out->data, numel(*out) * 4, s));
    VAE_TRY(launch_merge(*tile_out, to_box(&ob, *out), MergeRamps{*tile}, *out, s));
    if (flags & VAE_MERGE_FINALIZE) {
        AxisTiling ax[3];
        overlap_axes(*desc, ax);
        VAE_TRY(launch_merge_finalize(*out, ax[0], ax[1], ax[2], s));
    }
    return VAE_OK;
}

}  // extern "C"
