// Decode executor: a layer plan over caller-owned device weights and workspace.
//
// Mode A (patch-halo). On one GPU all patches share one activation tensor per layer, and each
// patch's halo is simply its neighbour's data in that tensor. Two ways to launch it:
//  - merged (VAE_LAUNCH_MERGED, the default): one launch per layer covers every patch box at once;
//    a GroupNorm's statistics come from that launch's blocks, which is the whole-tensor result;
//  - per patch (VAE_LAUNCH_PER_PATCH): every conv, GroupNorm pass and upsampling is launched once
//    per patch box, over that box only, as one rank of a patch split runs it. A GroupNorm's
//    statistics are formed per patch box (count, mean, M2) and merged across the patches with
//    Chan's update before any patch is normalised ("Add tiled VAE parallelism & extended model
//    support", PatchConv3d and PatchGroupNorm commit messages). Ops that need no box (the
//    per-position RMS norm, the whole-frame attention, the space-to-depth fold) stay one launch.
// Either way the final unpatchify places every patch's pixels disjointly, straight into `out`.
// Mode B (overlap-blend). The serial tiled decode of "[TRTLLM-14029][feat] LTX-2 tile-parallel VAE
// decode" (Description): one tile in flight. Each tile's latent box is cropped, decoded with its own
// borders and statistics, and blended into `out`, which is normalised after the last tile.
// Host work per call is integer geometry only; no host-built masks, no host-to-device copies.
#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "host.h"

struct vae_decoder {
    int32_t dtype = 0, act_dtype = 0, flags = 0, latent_c = 0, groups = 0;
    int32_t launch = VAE_LAUNCH_MERGED;   // patch-halo launches: merged or one per patch box
    int32_t clip = 0;    // patch-halo decodes in causal clips of this many latent frames (0: whole)
    float eps = 0.0f;
    std::vector<vae_layer_desc_t> layers;
    std::vector<const void*> ptrs;
    std::vector<const void*> packed;   // per entry of ptrs: packed copy of a conv weight or null
    bool timing = false;
    struct Rec {
        int32_t kind, layer, tile;
        double flops, bytes;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> events;
};

namespace vae {
namespace {

struct Shape {
    int64_t n, t, h, w, c;
    int32_t dtype;
    int64_t bytes() const { return n * t * h * w * c * elem_size(dtype); }
    int64_t frame_bytes() const { return n * h * w * c * elem_size(dtype); }
};

// Frames of headroom before every activation of a clip-by-clip decode: a causal conv's carried
// input frames go there.
constexpr int64_t kCarry = 2;

// Whether layer i is a conv that applies an fp32 input as split hi + lo bf16 operands.
bool conv_splits(int32_t flags, const vae_layer_desc_t* layers, int n, int i) {
    return (flags & VAE_DECODE_SPLIT_FP32_OPERANDS) && i >= 0 && i < n &&
           layers[i].op == VAE_OP_CONV && !layers[i].no_split;
}

// Whether layer i is a conv that takes fp16 operands (VAE_DECODE_F16_OPERANDS): a CONV on the
// matrix cores right after a RES whose convs also run there, or after a GN_SILU, in a plan that
// keeps fp32 activations (a bf16 stream has nothing finer to hand on). Its producer stores fp16.
// NEAREST ops between the producer and the conv only copy, so they pass fp16 values through.
bool conv_f16(int32_t dtype, int32_t act_dtype, int32_t flags, const vae_layer_desc_t* layers,
              int n, int i) {
    if (!(flags & VAE_DECODE_F16_OPERANDS) || dtype != VAE_DTYPE_BF16 ||
        act_dtype != VAE_DTYPE_F32 || i < 1 || i >= n)
        return false;
    const vae_layer_desc_t& l = layers[i];
    if ((l.op != VAE_OP_CONV && l.op != VAE_OP_CONV_DOWN) || l.cin % 32 || l.cout % 4)
        return false;
    int j = i - 1;
    while (j > 0 && layers[j].op == VAE_OP_NEAREST) --j;
    if (j > 0 && layers[j].op == VAE_OP_D2S) --j;       // the d2s its producing conv writes
    const vae_layer_desc_t& prev = layers[j];
    if (prev.op == VAE_OP_CONV)
        // a conv stores fp16 from a 2-byte input: the latent (plan dtype) or fp16 operands
        return !prev.f32_out && prev.cin % 32 == 0 && prev.cout % 4 == 0 &&
               (j == 0 || conv_f16(dtype, act_dtype, flags, layers, n, j));
    return ((prev.op == VAE_OP_RES || prev.op == VAE_OP_RES_RMS) && prev.cin % 32 == 0) ||
           prev.op == VAE_OP_GN_SILU || prev.op == VAE_OP_RMS_SILU;
}
// Whether the CONV at layer i stores fp16 for an fp16-operand conv it feeds (through its d2s and
// NEAREST copies).
bool conv_out_f16(int32_t dtype, int32_t act_dtype, int32_t flags,
                  const vae_layer_desc_t* layers, int n, int i) {
    int j = i + 1;
    if (j < n && layers[j].op == VAE_OP_D2S) ++j;
    while (j < n && layers[j].op == VAE_OP_NEAREST) ++j;
    return j < n && (layers[j].op == VAE_OP_CONV || layers[j].op == VAE_OP_CONV_DOWN) &&
           conv_f16(dtype, act_dtype, flags, layers, n, j);
}
// The conv (stride 1 or strided) that layer i feeds, past any NEAREST ops, or -1.
int fed_conv(const vae_layer_desc_t* layers, int n, int i) {
    int j = i + 1;
    while (j < n && layers[j].op == VAE_OP_NEAREST) ++j;
    return j < n && (layers[j].op == VAE_OP_CONV || layers[j].op == VAE_OP_CONV_DOWN) ? j : -1;
}
bool conv_f16(const vae_decoder& d, int i) {
    return conv_f16(d.dtype, d.act_dtype, d.flags, d.layers.data(), (int)d.layers.size(), i);
}

// Output dtype of the standalone GN_SILU at layer i: fp16 when the next layer is a conv with
// fp16 operands, the activation dtype when it is a conv that splits its fp32 input, else the conv
// operand dtype.
int32_t gn_silu_dtype(int32_t dtype, int32_t act_dtype, int32_t flags,
                      const vae_layer_desc_t* layers, int n, int i) {
    const int j = fed_conv(layers, n, i);
    if (j >= 0 && conv_f16(dtype, act_dtype, flags, layers, n, j)) return VAE_DTYPE_F16;
    return conv_splits(flags, layers, n, i + 1) ? act_dtype : dtype;
}
int32_t gn_silu_dtype(const vae_decoder& d, int i) {
    return gn_silu_dtype(d.dtype, d.act_dtype, d.flags, d.layers.data(), (int)d.layers.size(), i);
}

// Storage dtype of a residual block's output (layer i). When the next layer is a conv that rounds
// its input to the bf16 operand dtype anyway (bf16 weights on the matrix cores, no split), the
// block stores bf16 directly: the same rounding, done once at the store, with half the bytes.
// With fp16 operands for the next conv, the block stores fp16 (the one rounding that conv's
// operand gets).
// The first conv of a RES or RES_RMS block writes the tensor that only the block's second norm
// reads. With fp16 operands it is stored in fp16: the norm reads 2 bytes a value instead of 4,
// and the conv writes half as much.
// (The conv must run on the matrix cores, which hold the fp16 output path: Cin % 32 == 0.)
int32_t res_mid_dtype(const vae_decoder& d, int32_t width) {
    return (d.flags & VAE_DECODE_F16_OPERANDS) && d.dtype == VAE_DTYPE_BF16 &&
                   d.act_dtype == VAE_DTYPE_F32 && width % 32 == 0
               ? VAE_DTYPE_F16
               : d.act_dtype;
}

int32_t res_out_dtype(const vae_decoder& d, size_t i) {
    const int j = fed_conv(d.layers.data(), (int)d.layers.size(), (int)i);
    if (j >= 0 && conv_f16(d, j)) return VAE_DTYPE_F16;
    if (i + 1 < d.layers.size() && d.dtype == VAE_DTYPE_BF16 && d.layers[i].cin % 32 == 0) {
        const vae_layer_desc_t& n = d.layers[i + 1];
        if ((n.op == VAE_OP_CONV || n.op == VAE_OP_CONV_DOWN) &&
            !conv_splits(d.flags, d.layers.data(), (int)d.layers.size(), (int)i + 1) &&
            n.cin % 32 == 0 && n.cout % 4 == 0)
            return VAE_DTYPE_BF16;
    }
    return d.act_dtype;
}

// log2 of a power-of-two factor up to 16, else -1.
int32_t log2_of(int32_t f) {
    for (int32_t l = 0; l <= 4; ++l)
        if (f == (1 << l)) return l;
    return -1;
}

// Whether the op after layer i starts with a GroupNorm of layer i's output.
bool gn_follows(const vae_decoder& d, size_t i) {
    if (i + 1 >= d.layers.size()) return false;
    const int32_t op = d.layers[i + 1].op;
    return op == VAE_OP_RES || op == VAE_OP_GN_SILU;
}

// Number of device pointers each op consumes.
int ptrs_for(const vae_layer_desc_t& l) {
    switch (l.op) {
        case VAE_OP_CONV: return 2;
        case VAE_OP_CONV_DOWN: return 2;
        case VAE_OP_RES: return 8;
        case VAE_OP_GN_SILU: return 2;
        case VAE_OP_RES_RMS: return 8;
        case VAE_OP_RMS_SILU: return 2;
        case VAE_OP_ATTN: return 6;
        default: return 0;
    }
}

// Shape after each op, starting from the latent extents.
// `drop`: a causal depth-to-space drops its first st - 1 frames (false for the later clips of a
// clip-by-clip decode, which continue the sequence).
vae_status_t walk(const vae_decoder& d, Shape in, std::vector<Shape>* shapes, int* total_st,
                  int* total_sh, int* total_sw, bool drop = true) {
    Shape s = in;
    int st = 1, sh = 1, sw = 1;
    if (shapes) shapes->clear();
    for (size_t i = 0; i < d.layers.size(); ++i) {
        const vae_layer_desc_t& l = d.layers[i];
        switch (l.op) {
            case VAE_OP_CONV:
                s.c = l.cout;
                s.dtype = l.f32_out ? VAE_DTYPE_F32
                          : conv_out_f16(d.dtype, d.act_dtype, d.flags, d.layers.data(),
                                         (int)d.layers.size(), (int)i)
                              ? VAE_DTYPE_F16
                              : d.act_dtype;
                break;
            case VAE_OP_RES:
            case VAE_OP_RES_RMS:
                s.dtype = res_out_dtype(d, i);
                break;
            case VAE_OP_GN_SILU:
            case VAE_OP_RMS_SILU:
                s.dtype = gn_silu_dtype(d, (int)i);
                break;
            case VAE_OP_ATTN:
                s.dtype = VAE_DTYPE_F32;
                break;
            case VAE_OP_D2S:
                s.t = l.st * s.t - (drop ? l.st - 1 : 0);
                s.h *= l.sh;
                s.w *= l.sw;
                s.c /= (int64_t)l.st * l.sh * l.sw;
                st *= l.st;
                sh *= l.sh;
                sw *= l.sw;
                break;
            case VAE_OP_NEAREST:
                s.h *= l.sh;
                s.w *= l.sw;
                sh *= l.sh;
                sw *= l.sw;
                break;
            case VAE_OP_CONV_DOWN:
                if (s.h % l.sh || s.w % l.sw)
                    return fail(VAE_ERR_INVALID_ARG,
                                "a strided conv's input rows and columns must be whole strides",
                                s.h % l.sh ? 2 : 3, s.h % l.sh ? s.h : s.w, s.h % l.sh ? l.sh : l.sw);
                s.c = l.cout;
                s.dtype = l.f32_out ? VAE_DTYPE_F32 : d.act_dtype;
                s.t = (s.t - 1) / l.st + 1;
                s.h /= l.sh;   // (H + pt + pb - 3) / sh + 1 for whole strides and one row of padding
                s.w /= l.sw;
                break;
            case VAE_OP_S2D:
                {
                    vae_tensor_t g{};
                    g.n = s.n;
                    g.t = s.t;
                    g.h = s.h;
                    g.w = s.w;
                    g.c = s.c;
                    VAE_TRY(check_fold(g, l.st, l.sh, l.sw));
                }
                s.t = (s.t + l.st - 1) / l.st;
                s.h /= l.sh;
                s.w /= l.sw;
                s.c *= (int64_t)l.st * l.sh * l.sw;
                break;
            default:
                break;
        }
        if (shapes) shapes->push_back(s);
    }
    if (total_st) *total_st = st;
    if (total_sh) *total_sh = sh;
    if (total_sw) *total_sw = sw;
    return VAE_OK;
}

vae_tensor_t tensor_of(void* p, const Shape& s) {
    vae_tensor_t t{};
    t.data = p;
    t.dtype = s.dtype;
    t.n = s.n;
    t.t = s.t;
    t.h = s.h;
    t.w = s.w;
    t.c = s.c;
    return t;
}

Shape shape_of(const vae_tensor_t& t) { return Shape{t.n, t.t, t.h, t.w, t.c, t.dtype}; }

// Input-grid patch boxes scaled to an activation with cumulative spatial scale (ch, cw) and
// cumulative fold (fh, fw): rows b.h0 * ch / fh and so on. The division is exact: an encoder's
// patch bands are cut in whole multiples of its total fold (check_tiling refuses other bands),
// and a partial fold (fh, fw) divides the total one. `ok`, when given, is cleared if a division
// would not be exact.
BoxList scaled_boxes(const std::vector<Box>& latent_boxes, int64_t t, int ch, int cw, int fh = 1,
                     int fw = 1, bool* ok = nullptr) {
    BoxList bl;
    bl.n = (int32_t)latent_boxes.size();
    for (size_t i = 0; i < latent_boxes.size(); ++i) {
        const Box& b = latent_boxes[i];
        if (ok && ((int64_t)b.h0 * ch % fh || (int64_t)b.h1 * ch % fh ||
                   (int64_t)b.w0 * cw % fw || (int64_t)b.w1 * cw % fw))
            *ok = false;
        bl.b[i] = Box{0, (int32_t)t, b.h0 * ch / fh, b.h1 * ch / fh, b.w0 * cw / fw,
                      b.w1 * cw / fw};
    }
    return bl;
}

// Whether the plan has a space-to-depth fold (an encoder plan), and its total folds.
bool plan_folds(const vae_decoder& d, int32_t* ft = nullptr, int32_t* fh = nullptr,
                int32_t* fw = nullptr) {
    int32_t t = 1, h = 1, w = 1;
    bool any = false;
    for (const vae_layer_desc_t& l : d.layers)
        if (l.op == VAE_OP_S2D || l.op == VAE_OP_CONV_DOWN) {
            any = true;
            t *= l.st;
            h *= l.sh;
            w *= l.sw;
        }
    if (ft) *ft = t;
    if (fh) *fh = h;
    if (fw) *fw = w;
    return any;
}

struct Req {
    int64_t act = 0;      // bytes of the largest activation kept in a rotating buffer
    int64_t gn = 0;       // GroupNorm stats workspace
    int64_t parts = 0;    // per-patch GroupNorm moments (per-patch launches)
    int64_t splitk = 0;   // partial sums of a conv split over K (small launches)
    int64_t mr = 0;       // mean/rstd
    int64_t crop = 0;     // latent crop (mode B)
    int64_t tile = 0;     // one decoded tile, fp32 pixels (mode B)
    int64_t attn = 0;     // frame attention scratch
    int64_t carry = 0;    // carried input frames of every causal conv (clip-by-clip decodes)
    int64_t ab = 0;       // a GroupNorm's per-channel scale and shift (applied by the next conv)
};

// Requirements of one run of the plan on an input of shape `in` with patch boxes `boxes`.
// `headroom`: frames kept free before every activation held in a rotating buffer, and the
// carried frames of every causal conv (clip-by-clip decodes).
vae_status_t requirements(const vae_decoder& d, const Shape& in, const std::vector<Box>& boxes,
                          bool final_in_buffer, Req* r, int64_t headroom = 0) {
    auto held = [&](const Shape& x) { return x.bytes() + headroom * x.frame_bytes(); };
    auto carry = [&](const Shape& x) {   // a conv's two carried input frames (x: its input)
        if (headroom) r->carry += (int64_t)align_up((size_t)(kCarry * x.frame_bytes()), 256);
    };
    bool exact = true;   // every patch box scales to whole rows and columns of each activation
    const bool per_patch = d.launch == VAE_LAUNCH_PER_PATCH && boxes.size() > 1;
    std::vector<Shape> shapes;
    // a later clip keeps every frame of its depth-to-spaces: the larger shapes
    walk(d, in, &shapes, nullptr, nullptr, nullptr, headroom == 0);
    if (headroom) r->act = std::max(r->act, held(in));   // the clip's latent, copied in
    Shape cur = in;
    int ch = 1, cw = 1, fh = 1, fw = 1;
    for (size_t i = 0; i < d.layers.size(); ++i) {
        const vae_layer_desc_t& l = d.layers[i];
        const Shape& s = shapes[i];
        const bool last = i + 1 == d.layers.size();
        if (!last) r->act = std::max(r->act, held(s));
        if (last && final_in_buffer) r->tile = std::max(r->tile, s.bytes());
        if (l.op == VAE_OP_RES_RMS || l.op == VAE_OP_RMS_SILU) {
            Shape g = cur;
            g.dtype = l.op == VAE_OP_RES_RMS ? d.dtype : gn_silu_dtype(d, (int)i);
            r->act = std::max(r->act, std::max(held(cur), held(g)));
            if (l.op == VAE_OP_RES_RMS) {
                carry(g);    // conv1 and conv2 read bf16 norm outputs of cur's grid
                carry(g);
            }
        }
        if (l.op == VAE_OP_ATTN)
            r->attn = std::max<int64_t>(r->attn,
                                        (int64_t)attention_workspace(tensor_of(nullptr, cur)));
        if (l.op == VAE_OP_RES || l.op == VAE_OP_GN_SILU) {
            Shape g = cur;
            g.dtype = l.op == VAE_OP_RES ? d.dtype : gn_silu_dtype(d, (int)i);
            r->act = std::max(r->act, std::max(held(cur), held(g)));
            vae_tensor_t x = tensor_of(nullptr, cur);
            const BoxList bl = scaled_boxes(boxes, cur.t, ch, cw, fh, fw, &exact);
            r->gn = std::max<int64_t>(r->gn, (int64_t)gn_stats_workspace(x, bl, d.groups));
            if (per_patch)
                for (int b = 0; b < bl.n; ++b) {
                    BoxList one;
                    one.n = 1;
                    one.b[0] = bl.b[b];
                    r->gn = std::max<int64_t>(r->gn, (int64_t)gn_stats_workspace(x, one, d.groups));
                }
            r->parts = std::max<int64_t>(r->parts, (int64_t)bl.n * cur.n * d.groups * 3 *
                                                       (int64_t)sizeof(double));
            r->mr = std::max<int64_t>(r->mr, cur.n * d.groups * 2 * (int64_t)sizeof(float));
            r->ab = std::max<int64_t>(r->ab, cur.n * cur.c * 2 * (int64_t)sizeof(float));
        }
        // partials of GroupNorm statistics gathered by conv epilogues: over the whole grid, or
        // per patch box in rows holding every box's slots
        const bool next_gn = gn_follows(d, i);
        auto fused = [&](const Shape& xs, const Shape& ys, int32_t k) {
            const vae_tensor_t x = tensor_of(nullptr, xs);
            int64_t slots = 0;
            if (per_patch) {
                // xs is the conv's input grid; the boxes scale with it (nearest folds included)
                const BoxList bl = scaled_boxes(boxes, xs.t, ch, cw, fh, fw, &exact);
                for (int b = 0; b < bl.n; ++b)
                    slots += conv_gn_slots(x, ys.c, d.dtype, bl.b[b], d.groups, k, true);
            } else {
                slots = conv_gn_slots(x, ys.c, d.dtype, whole_box(x), d.groups, k, true);
            }
            r->gn = std::max<int64_t>(r->gn, ys.n * d.groups * slots * 3 * (int64_t)sizeof(double));
        };
        // scratch of convs split over K: the largest of the plan's launches, which run one at a
        // time
        auto split = [&](const Shape& xs, int64_t cout, bool split_fp32) {
            const vae_tensor_t x = tensor_of(nullptr, xs);
            BoxList bl;
            if (per_patch) {
                bl = scaled_boxes(boxes, xs.t, ch, cw, fh, fw, &exact);
            } else {
                bl.n = 1;
                bl.b[0] = whole_box(x);
            }
            for (int b = 0; b < bl.n; ++b) {
                const int32_t n = conv_split_count(x, cout, d.dtype, bl.b[b], split_fp32);
                r->splitk = std::max<int64_t>(
                    r->splitk, (int64_t)conv_split_bytes(x, cout, bl.b[b], n));
            }
        };
        if (l.op == VAE_OP_CONV) {
            split(cur, l.cout, conv_splits(d.flags, d.layers.data(), (int)d.layers.size(), (int)i));
            Shape xs = cur;              // its input, at most 4 bytes a value
            xs.dtype = VAE_DTYPE_F32;
            carry(xs);
        }
        if (l.op == VAE_OP_RES || l.op == VAE_OP_RES_RMS) {
            Shape xs = cur;
            xs.dtype = d.dtype;
            split(xs, l.cin, false);
        }
        if (l.op == VAE_OP_CONV && next_gn) fused(cur, s, 1);
        if (l.op == VAE_OP_CONV && i + 1 < d.layers.size() && d.layers[i + 1].op == VAE_OP_D2S &&
            gn_follows(d, i + 1)) {
            const vae_layer_desc_t& u = d.layers[i + 1];
            fused(cur, shapes[i + 1], u.st * u.sh * u.sw);
        }
        if (l.op == VAE_OP_RES) {
            // conv1 gathers the statistics of the block's second GroupNorm
            Shape xs = cur, ys = cur;
            xs.dtype = d.dtype;
            ys.dtype = res_mid_dtype(d, l.cin);
            fused(xs, ys, 1);
        }
        if ((l.op == VAE_OP_RES || l.op == VAE_OP_RES_RMS) && next_gn) {
            // conv2 gathers the statistics of the GroupNorm that reads the block's output
            Shape xs = cur;
            xs.dtype = d.dtype;
            fused(xs, s, 1);
        }
        if (l.op == VAE_OP_D2S || l.op == VAE_OP_NEAREST) {
            ch *= l.sh;
            cw *= l.sw;
        }
        if (l.op == VAE_OP_CONV_DOWN) {
            // y's grid folds by the strides; its epilogue may gather the next norm's statistics
            const vae_tensor_t y = tensor_of(nullptr, s);
            BoxList bl;
            if (per_patch) {
                bl = scaled_boxes(boxes, s.t, ch, cw, fh * l.sh, fw * l.sw, &exact);
            } else {
                bl.n = 1;
                bl.b[0] = whole_box(y);
            }
            int64_t slots = 0;
            if (next_gn)
                for (int b = 0; b < bl.n; ++b) slots += conv_strided_gn_slots(y, bl.b[b], d.groups);
            r->gn = std::max<int64_t>(r->gn, s.n * d.groups * slots * 3 * (int64_t)sizeof(double));
        }
        if (l.op == VAE_OP_S2D || l.op == VAE_OP_CONV_DOWN) {
            fh *= l.sh;
            fw *= l.sw;
        }
        cur = s;
    }
    if (!exact)
        return fail(VAE_ERR_INVALID_ARG, "patch bands do not fall on whole rows of every "
                                         "activation (an encoder's bands must be whole folds)");
    return VAE_OK;
}

struct Layout {
    size_t buf[3], gn, parts, splitk, mr, crop, tile, attn, carry, ab, status, total;
    int64_t act_bytes;
};

Layout layout_of(const Req& r) {
    Layout L{};
    size_t off = 0;
    const size_t act = align_up((size_t)r.act, 256);
    for (int i = 0; i < 3; ++i) {
        L.buf[i] = off;
        off += act;
    }
    L.gn = off;
    off += align_up((size_t)r.gn, 256);
    L.parts = off;
    off += align_up((size_t)r.parts, 256);
    L.splitk = off;
    off += align_up((size_t)r.splitk, 256);
    L.mr = off;
    off += align_up((size_t)r.mr, 256);
    L.crop = off;
    off += align_up((size_t)r.crop, 256);
    L.tile = off;
    off += align_up((size_t)r.tile, 256);
    L.attn = off;
    off += align_up((size_t)r.attn, 256);
    L.carry = off;
    off += align_up((size_t)r.carry, 256);
    L.ab = off;
    off += align_up((size_t)r.ab, 256);
    L.status = off;          // the decode's status word (vae_decode_status)
    off += 256;
    L.total = off;
    L.act_bytes = (int64_t)act;
    return L;
}

struct Runner {
    vae_decoder* d;
    hipStream_t s;
    uint8_t* ws;
    Layout L;
    int32_t tile;
    size_t ev;  // next event index

    vae_status_t mark(int32_t kind, int32_t layer, double flops, double bytes) {
        if (!d->timing) return VAE_OK;
        if (ev >= d->events.size()) {
            hipEvent_t e;
            VAE_HIP_CHECK(hipEventCreate(&e));
            d->events.push_back(e);
        }
        VAE_HIP_CHECK(hipEventRecord(d->events[ev], s));
        if (ev > 0) d->recs.push_back({kind, layer, tile, flops, bytes});
        ++ev;
        return VAE_OK;
    }

    bool stats_ready = false;  // mean/rstd already hold the statistics of the next GN's input
    bool pending_norm = false; // the next conv applies the norm whose scale and shift are formed
    // Clip-by-clip decode: activations keep kCarry frames of headroom, where every causal conv
    // puts its carried input frames (copies of frame 0 in the first clip).
    bool clips = false;
    bool first_clip = true;
    size_t carry_off = 0;      // next conv's carried frames in the workspace (per run)
    // The decode's status word in the workspace: set when a norm's statistics are not finite.
    uint32_t* status() { return reinterpret_cast<uint32_t*>(ws + L.status); }
    bool per_patch = false;    // launch every conv, GroupNorm pass and upsampling per patch box

    // Records an op of patch `patch` (-1: work shared by all patches, such as a merge of
    // statistics) in the timing.
    vae_status_t mark_patch(int32_t patch, int32_t kind, int32_t layer, double flops,
                            double bytes) {
        const int32_t keep = tile;
        if (per_patch) tile = patch;
        const vae_status_t st = mark(kind, layer, flops, bytes);
        tile = keep;
        return st;
    }

    // A GroupNorm + SiLU of x into y. Without y (nullptr) only its statistics (mean/rstd) and
    // the per-channel scale and shift are formed, for the conv that applies them as it stages x.
    vae_status_t gn(const vae_tensor_t& x, const vae_tensor_t* y, const BoxList& bl,
                    const void* gamma, const void* beta, int layer) {
        double* stats = reinterpret_cast<double*>(ws + L.gn);
        double* parts = reinterpret_cast<double*>(ws + L.parts);
        float* mr = reinterpret_cast<float*>(ws + L.mr);
        for (int i = 0; i < bl.n; ++i) {
            const Box& b = bl.b[i];
            if (b.t0 < 0 || b.h0 < 0 || b.w0 < 0 || b.t1 > x.t || b.h1 > x.h || b.w1 > x.w ||
                b.volume() <= 0)
                return fail(VAE_ERR_INVALID_ARG, "GroupNorm patch box outside the activation");
        }
        const bool fused = stats_ready;
        stats_ready = false;
        uint32_t* st = status();
        const double xe = (double)elem_size(x.dtype) * x.n * x.c;   // bytes per position
        auto scale_shift = [&]() {
            return launch_gn_scale_shift(mr, (int32_t)x.n, (int32_t)x.c, d->groups,
                                         static_cast<const float*>(gamma),
                                         static_cast<const float*>(beta), norm_ab(), s);
        };
        if (!per_patch) {
            if (!fused)
                VAE_TRY(launch_gn_stats(x, bl, d->groups, stats, nullptr, mr, d->eps, s, st));
            const double pos = (double)(x.t * x.h * x.w);
            if (!y) {
                VAE_TRY(scale_shift());
                return mark(VAE_KIND_GN, layer, 0.0, fused ? 0.0 : pos * xe);
            }
            // the patch boxes partition the tensor, so one apply launch covers them all
            VAE_TRY(launch_gn_apply(x, whole_box(x), d->groups, mr,
                                    static_cast<const float*>(gamma),
                                    static_cast<const float*>(beta), true, *y, s));
            const double ye = (double)elem_size(y->dtype) * y->n * y->c;
            return mark(VAE_KIND_GN, layer, 0.0, pos * ((fused ? 1.0 : 2.0) * xe + ye));
        }
        if (!fused) {
            // per-box (count, mean, M2), then one fixed-order Chan merge across the boxes
            for (int i = 0; i < bl.n; ++i) {
                BoxList one;
                one.n = 1;
                one.b[0] = bl.b[i];
                VAE_TRY(launch_gn_stats(x, one, d->groups, stats,
                                        parts + (int64_t)i * x.n * d->groups * 3, nullptr, d->eps,
                                        s, st));
                VAE_TRY(mark_patch(i, VAE_KIND_GN, layer, 0.0, (double)bl.b[i].volume() * xe));
            }
            VAE_TRY(launch_gn_combine(parts, bl.n, (int32_t)x.n, d->groups, d->eps, mr, s, st));
            VAE_TRY(mark_patch(-1, VAE_KIND_GN, layer, 0.0, 0.0));
        }
        if (!y) {   // one scale and shift for every patch: shared work
            VAE_TRY(scale_shift());
            return mark_patch(-1, VAE_KIND_GN, layer, 0.0, 0.0);
        }
        const double ye = (double)elem_size(y->dtype) * y->n * y->c;
        for (int i = 0; i < bl.n; ++i) {
            VAE_TRY(launch_gn_apply(x, bl.b[i], d->groups, mr, static_cast<const float*>(gamma),
                                    static_cast<const float*>(beta), true, *y, s));
            VAE_TRY(mark_patch(i, VAE_KIND_GN, layer, 0.0, (double)bl.b[i].volume() * (xe + ye)));
        }
        return VAE_OK;
    }

    float* norm_ab() { return reinterpret_cast<float*>(ws + L.ab); }

    // Whether the conv with weights d->ptrs[wi] in layer `layer` (cout conv channels) applies
    // the GroupNorm + SiLU of its input x while staging it (the norm's output is never written):
    // an MFMA conv with packed weights and no fp32 split, reading fp32, or fp16 with bf16 weights.
    bool fuse_norm(const vae_tensor_t& x, size_t wi, int layer, int64_t cout) const {
        if (!(d->flags & VAE_DECODE_NORM_IN_CONV) || !d->packed[wi] ||
            !conv_uses_mfma_c(x, cout, d->dtype) ||
            conv_splits(d->flags, d->layers.data(), (int)d->layers.size(), layer))
            return false;
        return x.dtype == VAE_DTYPE_F32 || (x.dtype == VAE_DTYPE_F16 && !conv_f16(*d, layer));
    }

    vae_status_t rms(const vae_tensor_t& x, const vae_tensor_t& y, const void* gamma,
                     const void* beta, int layer) {
        VAE_TRY(launch_rms_norm(x, d->eps, static_cast<const float*>(gamma),
                                static_cast<const float*>(beta), true, y, s, status()));
        return mark(VAE_KIND_RMS, layer, 0.0,
                    (double)numel(x) * elem_size(x.dtype) + (double)numel(y) * elem_size(y.dtype));
    }

    // `wi` indexes d->ptrs: the conv's weight, followed by its bias. With `gn_next` the conv's
    // epilogue also gathers the statistics of the GroupNorm that reads y. `up` (a D2S layer or
    // null) makes y the depth-to-space of the conv output, written by the conv's epilogue.
    // `lsh`, `lsw`: a nearest upsampling of x (log2 factors) that the conv reads while staging.
    // `bl`: the patch boxes in the conv's input grid; with per-patch launches the conv runs once
    // per box, and the statistics of all boxes land in one array that is merged once.
    // `in_ab`: the scale and shift of a GroupNorm + SiLU of x that the conv applies while staging
    // (fuse_norm), or null.
    vae_status_t conv(const vae_tensor_t& x, size_t wi, const vae_tensor_t* res,
                      const vae_tensor_t& y, int layer, bool gn_next, const BoxList& bl,
                      const vae_layer_desc_t* up = nullptr, int32_t lsh = 0, int32_t lsw = 0,
                      const float* in_ab = nullptr) {
        // a launch too small to fill the chip may split over K and take narrower channel tiles
        int32_t cf = VAE_CONV_SPLIT_K;
        if (conv_splits(d->flags, d->layers.data(), (int)d->layers.size(), layer))
            cf |= VAE_CONV_SPLIT_FP32;
        const void* w = d->ptrs[wi];
        if (d->packed[wi]) {
            // convs with fp16 operands were packed as fp16 (see vae_decoder_pack_weights); their
            // input is fp16, or the fp32 input of the norm they apply
            w = d->packed[wi];
            const bool f16w = in_ab ? conv_f16(*d, layer) : x.dtype == VAE_DTYPE_F16;
            cf |= f16w ? VAE_CONV_PACKED_F16_WEIGHTS : VAE_CONV_PACKED_WEIGHTS;
        }
        const int32_t k = up ? up->st * up->sh * up->sw : 1;
        const int64_t cout = y.c * k;
        // In a clip-by-clip decode x sits kCarry frames past the start of its buffer: put the
        // carried frames there (copies of frame 0 in the first clip, the causal padding) and run
        // the conv over the extended clip, writing only the clip's own frames.
        vae_tensor_t xe = x;
        int32_t t0 = 0, tdrop = -1;
        uint8_t* carry = nullptr;
        const int64_t fb = Shape{x.n, x.t, x.h, x.w, x.c, x.dtype}.frame_bytes();
        if (clips) {
            if (!conv_uses_mfma_c(x, cout, d->dtype))
                return fail(VAE_ERR_UNSUPPORTED, "a clip-by-clip decode runs its convs on the "
                                                 "matrix cores (bf16, 32k input channels)");
            uint8_t* head = static_cast<uint8_t*>(x.data) - kCarry * fb;
            carry = ws + L.carry + carry_off;
            carry_off += align_up((size_t)(kCarry * fb), 256);
            if (first_clip) {
                for (int64_t f = 0; f < kCarry; ++f)
                    VAE_TRY(launch_copy(head + f * fb, x.data, fb, s));
            } else {
                VAE_TRY(launch_copy(head, carry, kCarry * fb, s));
            }
            xe.data = head;
            xe.t = x.t + kCarry;
            t0 = (int32_t)kCarry;
            const int32_t st = up ? up->st : 1;
            tdrop = (int32_t)kCarry * st + (first_clip ? st - 1 : 0);
        }
        vae_tensor_t xl = xe;                      // the conv's input grid
        xl.h <<= lsh;
        xl.w <<= lsw;
        BoxList launches;                          // one launch per entry
        if (per_patch) {
            launches = bl;
        } else {
            launches.n = 1;
            launches.b[0] = whole_box(x);
            launches.b[0].h1 = (int32_t)xl.h;
            launches.b[0].w1 = (int32_t)xl.w;
        }
        for (int i = 0; i < launches.n; ++i) {    // the clip's own frames of the extended grid
            launches.b[i].t0 += t0;
            launches.b[i].t1 += t0;
        }
        int64_t slots[kMaxBoxes], total = 0;
        for (int i = 0; i < launches.n; ++i) {
            const Box& b = launches.b[i];
            if (b.t0 < 0 || b.h0 < 0 || b.w0 < 0 || b.t1 > xl.t || b.h1 > xl.h || b.w1 > xl.w ||
                b.volume() <= 0)
                return fail(VAE_ERR_INVALID_ARG, "conv patch box outside the activation");
            slots[i] = gn_next ? conv_gn_slots(xe, y.c, d->dtype, b, d->groups, k, true) : 0;
            total += slots[i];
        }
        double* part = reinterpret_cast<double*>(ws + L.gn);
        const double in_pos = (double)elem_size(x.dtype) * x.c * x.n;     // bytes per position
        const double out_pos = (double)elem_size(y.dtype) * y.c * k * y.n * (res ? 2.0 : 1.0);
        int64_t slot0 = 0;
        for (int i = 0; i < launches.n; ++i) {
            const Box& b = launches.b[i];
            ConvFuse fz{total > 0 ? part : nullptr, d->groups, up ? up->st : 1, up ? up->sh : 1,
                        up ? up->sw : 1, lsh, lsw};
            fz.slot0 = slot0;
            fz.slot_stride = total;
            fz.tdrop = tdrop;
            fz.in_ab = in_ab;
            // a launch too small to fill the chip splits its K dimension over the scratch
            fz.splits = conv_split_count(xl, cout, d->dtype, b, (cf & VAE_CONV_SPLIT_FP32) != 0);
            if (fz.splits > 1) fz.part = reinterpret_cast<float*>(ws + L.splitk);
            slot0 += slots[i];
            VAE_TRY(launch_conv3d(xe, w, d->dtype, static_cast<const float*>(d->ptrs[wi + 1]),
                                  res, y, b, cf, s, &fz));
            const double pos = (double)b.volume() * x.n;
            const double flops = 2.0 * 27.0 * (double)x.c * (double)cout * pos;
            // input read once (at its own resolution), output (and residual) once
            const double bytes = pos / x.n / (double)(1 << (lsh + lsw)) * in_pos +
                                 (double)b.volume() * out_pos;
            VAE_TRY(mark_patch(i, VAE_KIND_CONV, layer, flops, bytes));
        }
        if (clips)   // the last kCarry frames of the extended input carry on to the next clip
            VAE_TRY(launch_copy(carry, static_cast<uint8_t*>(xe.data) + x.t * fb, kCarry * fb, s));
        if (total > 0) {
            // merged into mean/rstd here (all patches, in a fixed order); timed as shared work
            VAE_TRY(launch_gn_finalize_slots(part, total, (int32_t)y.n, d->groups, d->eps,
                                             reinterpret_cast<float*>(ws + L.mr), s, status()));
            if (per_patch) VAE_TRY(mark_patch(-1, VAE_KIND_GN, layer, 0.0, 0.0));
            stats_ready = true;
        }
        return VAE_OK;
    }

    // A strided conv (an encoder's downsampler) into y, over y's whole grid or per patch box (`bl`,
    // boxes of y); with `gn_next` its epilogue gathers the next GroupNorm's statistics.
    vae_status_t conv_down(const vae_tensor_t& x, size_t wi, const vae_tensor_t& y, int layer,
                           const vae_layer_desc_t& l, bool gn_next, const BoxList& bl) {
        const void* w = d->ptrs[wi];
        int32_t cf = 0;
        if (d->packed[wi]) {
            w = d->packed[wi];
            cf = x.dtype == VAE_DTYPE_F16 ? VAE_CONV_PACKED_F16_WEIGHTS : VAE_CONV_PACKED_WEIGHTS;
        }
        const int32_t before = l.pad == VAE_PAD_AROUND ? 1 : 0;
        const StrideGeom g{l.st, l.sh, l.sw, before, before};
        BoxList launches;
        if (per_patch) {
            launches = bl;
        } else {
            launches.n = 1;
            launches.b[0] = whole_box(y);
        }
        const bool fuse = gn_next && conv_strided_uses_mfma(x, y.c, d->dtype, cf, g);
        int64_t slots[kMaxBoxes], total = 0;
        for (int i = 0; i < launches.n; ++i) {
            const Box& b = launches.b[i];
            if (b.t0 < 0 || b.h0 < 0 || b.w0 < 0 || b.t1 > y.t || b.h1 > y.h || b.w1 > y.w ||
                b.volume() <= 0)
                return fail(VAE_ERR_INVALID_ARG, "strided conv patch box outside the activation");
            slots[i] = fuse ? conv_strided_gn_slots(y, b, d->groups) : 0;
            total += slots[i];
        }
        double* part = reinterpret_cast<double*>(ws + L.gn);
        int64_t slot0 = 0;
        for (int i = 0; i < launches.n; ++i) {
            const Box& b = launches.b[i];
            ConvFuse fz{total > 0 ? part : nullptr, d->groups, 1, 1, 1};
            fz.slot0 = slot0;
            fz.slot_stride = total;
            slot0 += slots[i];
            VAE_TRY(launch_conv3d_strided(x, w, d->dtype, static_cast<const float*>(d->ptrs[wi + 1]),
                                          nullptr, y, b, g, cf, s, &fz));
            const double pos = (double)b.volume() * y.n;
            const double flops = 2.0 * 27.0 * (double)x.c * (double)y.c * pos;
            const double bytes = pos * (double)l.st * l.sh * l.sw * x.c * elem_size(x.dtype) +
                                 pos * (double)y.c * elem_size(y.dtype);
            VAE_TRY(mark_patch(i, VAE_KIND_CONV, layer, flops, bytes));
        }
        if (total > 0) {
            VAE_TRY(launch_gn_finalize_slots(part, total, (int32_t)y.n, d->groups, d->eps,
                                             reinterpret_cast<float*>(ws + L.mr), s, status()));
            if (per_patch) VAE_TRY(mark_patch(-1, VAE_KIND_GN, layer, 0.0, 0.0));
            stats_ready = true;
        }
        return VAE_OK;
    }

    // A standalone depth-to-space or nearest upsampling: over the whole tensor, or per patch box
    // (boxes in x's grid).
    vae_status_t upsample(const vae_tensor_t& x, const BoxList& bl, int mode, int32_t st,
                          int32_t sh, int32_t sw, const vae_tensor_t& y, int layer) {
        const double e = (double)elem_size(x.dtype) * x.c * x.n;
        const double k = (double)sh * sw * (mode == VAE_UPSAMPLE_D2S ? 1.0 / (sh * sw) : 1.0);
        if (!per_patch) {
            VAE_TRY(launch_upsample(x, whole_box(x), mode, st, sh, sw, y, s));
            return mark(VAE_KIND_UPSAMPLE, layer, 0.0,
                        (double)numel(x) * elem_size(x.dtype) +
                            (double)numel(y) * elem_size(y.dtype));
        }
        for (int i = 0; i < bl.n; ++i) {
            VAE_TRY(launch_upsample(x, bl.b[i], mode, st, sh, sw, y, s));
            VAE_TRY(mark_patch(i, VAE_KIND_UPSAMPLE, layer, 0.0,
                               (double)bl.b[i].volume() * e * (1.0 + k)));
        }
        return VAE_OK;
    }

    // Run the whole plan on `in`; the last op writes `final_out`.
    vae_status_t run(const vae_tensor_t& in, const std::vector<Box>& boxes,
                     const vae_tensor_t& final_out) {
        std::vector<Shape> shapes;
        VAE_TRY(walk(*d, shape_of(in), &shapes, nullptr, nullptr, nullptr,
                     !clips || first_clip));
        stats_ready = false;
        pending_norm = false;
        carry_off = 0;
        vae_tensor_t cur = in;
        int cur_buf = -1;  // -1: the caller's input, never written
        int ch = 1, cw = 1, fh = 1, fw = 1;
        int32_t near_lsh = 0, near_lsw = 0;   // a nearest upsampling the next conv reads
        size_t p = 0;
        // a buffer's tensor; in a clip-by-clip decode it starts kCarry frames into the buffer
        auto buf = [&](int i, const Shape& sh) {
            return tensor_of(ws + L.buf[i] + (clips ? kCarry * sh.frame_bytes() : 0), sh);
        };
        if (clips) {
            // the clip's latent goes into a buffer too, so that its first conv has headroom
            vae_tensor_t c = buf(0, shape_of(in));
            VAE_TRY(launch_copy(c.data, in.data, shape_of(in).bytes(), s));
            cur = c;
            cur_buf = 0;
        }
        auto free_buf = [&](int avoid1, int avoid2) {
            for (int i = 0; i < 3; ++i)
                if (i != avoid1 && i != avoid2) return i;
            return -1;
        };
        for (size_t li = 0; li < d->layers.size(); ++li) {
            const vae_layer_desc_t& l = d->layers[li];
            const bool last = li + 1 == d->layers.size();
            const Shape& os = shapes[li];
            const int layer = (int)li;
            if (l.op == VAE_OP_CONV) {
                // a depth-to-space right after the conv is done by the conv's epilogue
                const bool fuse_up = li + 1 < d->layers.size() &&
                                     d->layers[li + 1].op == VAE_OP_D2S &&
                                     conv_uses_mfma_c(cur, l.cout, d->dtype);
                const size_t lo = fuse_up ? li + 1 : li;
                const bool out_last = lo + 1 == d->layers.size();
                const int nb = free_buf(cur_buf, -1);
                vae_tensor_t y = out_last ? final_out : buf(nb, shapes[lo]);
                // ch, cw already hold a folded nearest upsampling: boxes in the conv's grid
                const BoxList cb = scaled_boxes(boxes, cur.t, ch, cw, fh, fw);
                VAE_TRY(conv(cur, p, nullptr, y, layer, gn_follows(*d, lo), cb,
                             fuse_up ? &d->layers[li + 1] : nullptr, near_lsh, near_lsw,
                             pending_norm ? norm_ab() : nullptr));
                near_lsh = near_lsw = 0;
                pending_norm = false;
                p += 2;
                cur = y;
                cur_buf = out_last ? -2 : nb;
                if (fuse_up) {
                    ch *= d->layers[li + 1].sh;
                    cw *= d->layers[li + 1].sw;
                    li = lo;
                }
            } else if (l.op == VAE_OP_RES) {
                // x -> GN1 -> t1 -> conv1 -> t2 -> GN2 -> t1 -> conv2 (+ x) -> t2
                // (a norm that its conv applies while staging writes no t1: the conv reads x or
                // t2 itself, and y then goes to b1)
                const BoxList bl = scaled_boxes(boxes, cur.t, ch, cw, fh, fw);
                const int b1 = free_buf(cur_buf, -1);
                const int b2 = free_buf(cur_buf, b1);
                Shape gs = shape_of(cur), as = shape_of(cur);
                gs.dtype = d->dtype;
                as.dtype = res_mid_dtype(*d, l.cin);
                vae_tensor_t t1 = buf(b1, gs), t2 = buf(b2, as);
                const bool f1 = fuse_norm(cur, p + 2, layer, l.cin);
                VAE_TRY(gn(cur, f1 ? nullptr : &t1, bl, d->ptrs[p], d->ptrs[p + 1], layer));
                VAE_TRY(conv(f1 ? cur : t1, p + 2, nullptr, t2, layer, true, bl, nullptr, 0, 0,
                             f1 ? norm_ab() : nullptr));
                const bool f2 = fuse_norm(t2, p + 6, layer, l.cin);
                VAE_TRY(gn(t2, f2 ? nullptr : &t1, bl, d->ptrs[p + 4], d->ptrs[p + 5], layer));
                Shape ys = as;
                ys.dtype = res_out_dtype(*d, li);
                const int yb = f2 ? b1 : b2;        // the buffer conv2 does not read
                vae_tensor_t y = last ? final_out : buf(yb, ys);
                VAE_TRY(conv(f2 ? t2 : t1, p + 6, &cur, y, layer, gn_follows(*d, li), bl, nullptr, 0,
                             0, f2 ? norm_ab() : nullptr));
                p += 8;
                cur = y;
                cur_buf = last ? -2 : yb;
            } else if (l.op == VAE_OP_RES_RMS) {
                // x -> RMS1 -> t1 -> conv1 -> t2 -> RMS2 -> t1 -> conv2 (+ x) -> t2
                const BoxList bl = scaled_boxes(boxes, cur.t, ch, cw, fh, fw);
                const int b1 = free_buf(cur_buf, -1);
                const int b2 = free_buf(cur_buf, b1);
                Shape gs = shape_of(cur), as = shape_of(cur);
                gs.dtype = d->dtype;
                as.dtype = res_mid_dtype(*d, l.cin);
                vae_tensor_t t1 = buf(b1, gs), t2 = buf(b2, as);
                stats_ready = false;
                VAE_TRY(rms(cur, t1, d->ptrs[p], d->ptrs[p + 1], layer));
                VAE_TRY(conv(t1, p + 2, nullptr, t2, layer, false, bl));
                VAE_TRY(rms(t2, t1, d->ptrs[p + 4], d->ptrs[p + 5], layer));
                Shape ys = as;
                ys.dtype = res_out_dtype(*d, li);
                vae_tensor_t y = last ? final_out : buf(b2, ys);
                VAE_TRY(conv(t1, p + 6, &cur, y, layer, gn_follows(*d, li), bl));
                p += 8;
                cur = y;
                cur_buf = last ? -2 : b2;
            } else if (l.op == VAE_OP_RMS_SILU) {
                vae_tensor_t y;
                int nb = cur_buf;
                Shape gs = shape_of(cur);
                gs.dtype = gn_silu_dtype(*d, layer);
                if (last) {
                    y = final_out;
                    nb = -2;
                } else if (cur_buf < 0 || cur.dtype != gs.dtype) {
                    nb = free_buf(cur_buf, -1);
                    y = buf(nb, gs);
                } else {
                    y = cur;  // in place
                }
                stats_ready = false;
                VAE_TRY(rms(cur, y, d->ptrs[p], d->ptrs[p + 1], layer));
                p += 2;
                cur = y;
                cur_buf = nb;
            } else if (l.op == VAE_OP_ATTN) {
                const int nb = free_buf(cur_buf, -1);
                vae_tensor_t y = last ? final_out : buf(nb, os);
                stats_ready = false;
                VAE_TRY(launch_frame_attention(
                    cur, d->eps, static_cast<const float*>(d->ptrs[p]),
                    static_cast<const float*>(d->ptrs[p + 1]), d->ptrs[p + 2],
                    static_cast<const float*>(d->ptrs[p + 3]), d->ptrs[p + 4],
                    static_cast<const float*>(d->ptrs[p + 5]), y, ws + L.attn, s));
                const double hw = (double)cur.h * cur.w, pos = (double)positions(cur);
                const double c = (double)cur.c;
                VAE_TRY(mark(VAE_KIND_ATTN, layer, 2.0 * pos * c * c * 4.0 + 4.0 * pos * hw * c,
                             0.0));
                p += 6;
                cur = y;
                cur_buf = last ? -2 : nb;
            } else if (l.op == VAE_OP_GN_SILU && !last && d->layers[li + 1].op == VAE_OP_CONV &&
                       fuse_norm(cur, p + 2, layer + 1, d->layers[li + 1].cout)) {
                // the next conv applies the norm while staging its input: statistics, scale and
                // shift only
                const BoxList bl = scaled_boxes(boxes, cur.t, ch, cw, fh, fw);
                VAE_TRY(gn(cur, nullptr, bl, d->ptrs[p], d->ptrs[p + 1], layer));
                p += 2;
                pending_norm = true;
            } else if (l.op == VAE_OP_GN_SILU) {
                const BoxList bl = scaled_boxes(boxes, cur.t, ch, cw, fh, fw);
                vae_tensor_t y;
                int nb = cur_buf;
                Shape gs = shape_of(cur);
                gs.dtype = gn_silu_dtype(*d, layer);
                if (last) {
                    y = final_out;
                    nb = -2;
                } else if (cur_buf < 0 || cur.dtype != gs.dtype) {
                    nb = free_buf(cur_buf, -1);
                    y = buf(nb, gs);
                } else {
                    y = cur;  // in place
                }
                VAE_TRY(gn(cur, &y, bl, d->ptrs[p], d->ptrs[p + 1], layer));
                p += 2;
                cur = y;
                cur_buf = nb;
            } else if (l.op == VAE_OP_NEAREST && !last && d->layers[li + 1].op == VAE_OP_CONV &&
                       conv_uses_mfma_c(cur, d->layers[li + 1].cout, d->dtype) &&
                       log2_of(l.sh) >= 0 && log2_of(l.sw) >= 0 &&
                       near_lsh + log2_of(l.sh) <= 4 && near_lsw + log2_of(l.sw) <= 4) {
                // a nearest upsampling feeding an MFMA conv: the conv reads it while staging its
                // input tile, so the upsampled tensor is never written
                near_lsh += log2_of(l.sh);
                near_lsw += log2_of(l.sw);
                ch *= l.sh;
                cw *= l.sw;
            } else if (l.op == VAE_OP_CONV_DOWN) {
                const int nb = free_buf(cur_buf, -1);
                vae_tensor_t y = last ? final_out : buf(nb, os);
                fh *= l.sh;   // y's grid
                fw *= l.sw;
                VAE_TRY(conv_down(cur, p, y, layer, l, gn_follows(*d, li),
                                  scaled_boxes(boxes, y.t, ch, cw, fh, fw)));
                p += 2;
                cur = y;
                cur_buf = last ? -2 : nb;
            } else if (l.op == VAE_OP_S2D) {
                const int nb = free_buf(cur_buf, -1);
                vae_tensor_t y = last ? final_out : buf(nb, os);
                VAE_TRY(launch_space_to_depth(cur, l.st, l.sh, l.sw, y, s));
                VAE_TRY(mark(VAE_KIND_UPSAMPLE, layer, 0.0,
                             (double)numel(cur) * elem_size(cur.dtype) +
                                 (double)numel(y) * elem_size(y.dtype)));
                fh *= l.sh;
                fw *= l.sw;
                cur = y;
                cur_buf = last ? -2 : nb;
            } else {  // D2S / NEAREST
                if (clips && l.op == VAE_OP_D2S && l.st > 1)
                    return fail(VAE_ERR_UNSUPPORTED,
                                "a clip-by-clip decode needs its temporal depth-to-space fused into "
                                "a matrix-core conv");
                const int nb = free_buf(cur_buf, -1);
                vae_tensor_t y = last ? final_out : buf(nb, os);
                const int mode = l.op == VAE_OP_D2S ? VAE_UPSAMPLE_D2S : VAE_UPSAMPLE_NEAREST;
                const int st = l.op == VAE_OP_D2S ? l.st : 1;
                VAE_TRY(upsample(cur, scaled_boxes(boxes, cur.t, ch, cw, fh, fw), mode, st, l.sh,
                                 l.sw, y, layer));
                ch *= l.sh;
                cw *= l.sw;
                cur = y;
                cur_buf = last ? -2 : nb;
            }
        }
        return VAE_OK;
    }
};

vae_status_t plan_output(const vae_decoder& d, const vae_tiling_desc_t& desc, Shape* out,
                         int* st, int* sh, int* sw) {
    Shape in{desc.n, desc.t, desc.h, desc.w, d.latent_c, d.dtype};
    std::vector<Shape> shapes;
    VAE_TRY(walk(d, in, &shapes, st, sh, sw));
    *out = shapes.back();
    return VAE_OK;
}

// Whether a decode runs clip by clip: a patch-halo decode longer than the decoder's clip.
bool clipped(const vae_decoder& d, const vae_tiling_desc_t& desc) {
    return d.clip > 0 && desc.mode == VAE_TILING_PATCH_HALO && desc.t > d.clip;
}

vae_status_t size_for(const vae_decoder& d, const vae_tiling_desc_t& desc, Layout* L,
                      std::vector<vae_tile_t>* tiles) {
    VAE_TRY(check_tiling(&desc));
    int st, sh, sw;
    Shape out;
    VAE_TRY(plan_output(d, desc, &out, &st, &sh, &sw));
    if (st != desc.scale_t || sh != desc.scale_h || sw != desc.scale_w)
        return fail(VAE_ERR_INVALID_ARG, "tiling scales do not match the decoder plan");
    int32_t ft, fh, fw;
    const bool folds = plan_folds(d, &ft, &fh, &fw);
    const bool untiled = desc.mode == VAE_TILING_PATCH_HALO && desc.patches_h == 1 &&
                         desc.patches_w == 1 && !encodes(desc);
    if (folds && !untiled &&
        (!encodes(desc) || std::max(desc.down_t, 1) != ft || std::max(desc.down_h, 1) != fh ||
         std::max(desc.down_w, 1) != fw))
        return fail(VAE_ERR_INVALID_ARG,
                    "an encoder (a plan with space-to-depth folds) is tiled with down_* = its "
                    "folds, or runs untiled (1 x 1 patches, no down_*)");
    if (!folds && encodes(desc))
        return fail(VAE_ERR_INVALID_ARG, "down_* is for plans with space-to-depth folds");
    if (desc.mode == VAE_TILING_PATCH_HALO && (int64_t)desc.patches_h * desc.patches_w > kMaxBoxes)
        return fail(VAE_ERR_UNSUPPORTED, "the decoder takes at most 16 patches", -1,
                    (int64_t)desc.patches_h * desc.patches_w, -1, 1);
    *tiles = make_tiles(desc);
    Req r;
    if (desc.mode == VAE_TILING_PATCH_HALO) {
        std::vector<Box> boxes;
        for (const vae_tile_t& t : *tiles)
            boxes.push_back(Box{t.latent.t0, t.latent.t1, t.latent.h0, t.latent.h1, t.latent.w0,
                                t.latent.w1});
        if (clipped(d, desc))   // sized for one clip without the frame drop, plus headroom
            VAE_TRY(requirements(d, Shape{desc.n, d.clip, desc.h, desc.w, d.latent_c, d.dtype},
                                 boxes, false, &r, kCarry));
        else
            VAE_TRY(requirements(d, Shape{desc.n, desc.t, desc.h, desc.w, d.latent_c, d.dtype},
                                 boxes, false, &r));
    } else {
        for (const vae_tile_t& t : *tiles) {
            Shape in{desc.n, t.latent.t1 - t.latent.t0, t.latent.h1 - t.latent.h0,
                     t.latent.w1 - t.latent.w0, d.latent_c, d.dtype};
            std::vector<Box> one{Box{0, (int32_t)in.t, 0, (int32_t)in.h, 0, (int32_t)in.w}};
            VAE_TRY(requirements(d, in, one, true, &r));
            r.crop = std::max(r.crop, in.bytes());
        }
    }
    *L = layout_of(r);
    return VAE_OK;
}

// Visit every conv of the plan: fn(ptr index of its weight, cin, cout, fp16 operands).
template <typename F>
void for_each_conv(const vae_decoder& d, F fn) {
    size_t p = 0;
    for (size_t i = 0; i < d.layers.size(); ++i) {
        const vae_layer_desc_t& l = d.layers[i];
        if (l.op == VAE_OP_CONV || l.op == VAE_OP_CONV_DOWN)
            fn(p, l.cin, l.cout, conv_f16(d, (int)i));
        if (l.op == VAE_OP_RES || l.op == VAE_OP_RES_RMS) {
            fn(p + 2, l.cin, l.cin, false);
            fn(p + 6, l.cin, l.cin, false);
        }
        p += ptrs_for(l);
    }
}

// Convs that run on the MFMA path (bf16 weights, Cin % 32 == 0, Cout % 4 == 0) are packable.
bool packable(const vae_decoder& d, int32_t cin, int32_t cout) {
    return d.dtype == VAE_DTYPE_BF16 && cin % 32 == 0 && cout % 4 == 0;
}

}  // namespace
}  // namespace vae

using namespace vae;

extern "C" {

VAE_API vae_status_t vae_decoder_create(const vae_decoder_spec_t* spec,
                                        const void* const* params, int32_t n_ptrs,
                                        vae_decoder_t** out) {
    clear_error();
    if (!spec || !out) return fail(VAE_ERR_INVALID_ARG, "spec or out is NULL");
    *out = nullptr;
    if (spec->dtype != VAE_DTYPE_BF16 && spec->dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_INVALID_ARG, "unknown plan dtype");
    if (spec->act_dtype != VAE_DTYPE_BF16 && spec->act_dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_INVALID_ARG, "unknown activation dtype");
    // bf16 activation storage rounds every op's output once more (about 40 extra roundings in
    // the LTX-2-shaped plan) and misses the 2e-2 max-abs bar of a bf16 decode: refused.
    if (spec->act_dtype != VAE_DTYPE_F32)
        return fail(VAE_ERR_UNSUPPORTED, "activations between ops are stored in fp32 "
                                         "(act_dtype must be VAE_DTYPE_F32)");
    if (spec->flags &
        ~(VAE_DECODE_SPLIT_FP32_OPERANDS | VAE_DECODE_F16_OPERANDS | VAE_DECODE_NORM_IN_CONV))
        return fail(VAE_ERR_INVALID_ARG, "unknown decoder flags");
    if ((spec->flags & VAE_DECODE_SPLIT_FP32_OPERANDS) && (spec->flags & VAE_DECODE_F16_OPERANDS))
        return fail(VAE_ERR_INVALID_ARG, "give one of the split and fp16 operand flags");
    if (spec->latent_channels < 1 || spec->groups < 1 || !(spec->eps >= 0.0f))
        return fail(VAE_ERR_INVALID_ARG, "latent_channels and groups must be >= 1, eps >= 0");
    if (spec->n_layers < 1 || !spec->layers) return fail(VAE_ERR_INVALID_ARG, "empty layer plan");
    int64_t c = spec->latent_channels;
    int32_t act = spec->dtype;
    int need = 0;
    for (int i = 0; i < spec->n_layers; ++i) {
        const vae_layer_desc_t& l = spec->layers[i];
        switch (l.op) {
            case VAE_OP_CONV:
                if (l.cin != c || l.cout < 1)
                    return fail(VAE_ERR_INVALID_ARG, "conv channels do not chain", 4, l.cin, -1, c);
                c = l.cout;
                act = l.f32_out ? VAE_DTYPE_F32 : spec->act_dtype;
                break;
            case VAE_OP_RES:
                if (l.cin != c) return fail(VAE_ERR_INVALID_ARG, "res width does not chain");
                if (act != spec->act_dtype)
                    return fail(VAE_ERR_UNSUPPORTED,
                                "a residual block input must have the activation dtype");
                if (c % spec->groups)
                    return fail(VAE_ERR_UNSUPPORTED, "width not divisible by groups", 4, c,
                                spec->groups);
                break;
            case VAE_OP_GN_SILU:
                if (c % spec->groups)
                    return fail(VAE_ERR_UNSUPPORTED, "width not divisible by groups", 4, c,
                                spec->groups);
                act = gn_silu_dtype(spec->dtype, spec->act_dtype, spec->flags, spec->layers,
                                    spec->n_layers, i);
                break;
            case VAE_OP_RES_RMS:
                if (l.cin != c) return fail(VAE_ERR_INVALID_ARG, "res width does not chain");
                if (act != spec->act_dtype)
                    return fail(VAE_ERR_UNSUPPORTED,
                                "a residual block input must have the activation dtype");
                if (!rms_shape_supported(c))
                    return fail(VAE_ERR_UNSUPPORTED, "rms norm width", 4, c, 8);
                break;
            case VAE_OP_RMS_SILU:
                if (!rms_shape_supported(c))
                    return fail(VAE_ERR_UNSUPPORTED, "rms norm width", 4, c, 8);
                act = gn_silu_dtype(spec->dtype, spec->act_dtype, spec->flags, spec->layers,
                                    spec->n_layers, i);
                break;
            case VAE_OP_ATTN:
                if (l.cin != c) return fail(VAE_ERR_INVALID_ARG, "attention width does not chain");
                if (spec->dtype != VAE_DTYPE_BF16 || spec->act_dtype != VAE_DTYPE_F32 ||
                    act != VAE_DTYPE_F32)
                    return fail(VAE_ERR_UNSUPPORTED,
                                "attention needs bf16 weights and fp32 activations");
                if (!attention_shape_supported(c))
                    return fail(VAE_ERR_UNSUPPORTED, "attention width", 4, c, 32);
                break;
            case VAE_OP_D2S: {
                if (l.st < 1 || l.sh < 1 || l.sw < 1)
                    return fail(VAE_ERR_INVALID_ARG, "d2s factors must be >= 1");
                const int64_t k = (int64_t)l.st * l.sh * l.sw;
                if (c % k) return fail(VAE_ERR_INVALID_ARG, "d2s: channels not divisible", 4, c, k);
                c /= k;
                break;
            }
            case VAE_OP_NEAREST:
                if (l.sh < 1 || l.sw < 1)
                    return fail(VAE_ERR_INVALID_ARG, "nearest factors must be >= 1");
                break;
            case VAE_OP_CONV_DOWN:
                if (l.cin != c || l.cout < 1)
                    return fail(VAE_ERR_INVALID_ARG, "conv channels do not chain", 4, l.cin, -1, c);
                if (l.st < 1 || l.st > 2 || l.sh < 1 || l.sh > 2 || l.sh != l.sw)
                    return fail(VAE_ERR_UNSUPPORTED, "a strided conv in a plan takes strides "
                                                     "st, sh = sw of 1 or 2");
                if (l.pad != VAE_PAD_AROUND && l.pad != VAE_PAD_AFTER)
                    return fail(VAE_ERR_INVALID_ARG, "unknown strided conv padding");
                if (l.pad == VAE_PAD_AFTER && l.sh != 2)
                    return fail(VAE_ERR_UNSUPPORTED, "padding after the image goes with stride 2 "
                                                     "(it would shrink a stride-1 axis)");
                c = l.cout;
                act = l.f32_out ? VAE_DTYPE_F32 : spec->act_dtype;
                break;
            case VAE_OP_S2D:
                if (l.st < 1 || l.sh < 1 || l.sw < 1)
                    return fail(VAE_ERR_INVALID_ARG, "s2d factors must be >= 1");
                c *= (int64_t)l.st * l.sh * l.sw;
                break;
            default:
                return fail(VAE_ERR_INVALID_ARG, "unknown op in layer plan");
        }
        need += ptrs_for(l);
    }
    if (act != VAE_DTYPE_F32)
        return fail(VAE_ERR_UNSUPPORTED, "the plan must end in fp32 (fp32 activations or f32_out)");
    if (n_ptrs != need || (need > 0 && !params))
        return fail(VAE_ERR_INVALID_ARG, "parameter pointer count does not match the plan", -1,
                    n_ptrs, -1, need);
    int p = 0;
    for (int i = 0; i < spec->n_layers; ++i) {
        const vae_layer_desc_t& l = spec->layers[i];
        if ((l.op == VAE_OP_CONV || l.op == VAE_OP_CONV_DOWN) && !params[p])
            return fail(VAE_ERR_INVALID_ARG, "conv weight pointer is NULL");
        if ((l.op == VAE_OP_RES || l.op == VAE_OP_RES_RMS) && (!params[p + 2] || !params[p + 6]))
            return fail(VAE_ERR_INVALID_ARG, "res conv weight pointer is NULL");
        if (l.op == VAE_OP_ATTN && (!params[p + 2] || !params[p + 4]))
            return fail(VAE_ERR_INVALID_ARG, "attention weight pointer is NULL");
        p += ptrs_for(l);
    }
    vae_decoder* d = new (std::nothrow) vae_decoder();
    if (!d) return fail(VAE_ERR_INVALID_ARG, "out of host memory");
    d->dtype = spec->dtype;
    d->act_dtype = spec->act_dtype;
    d->flags = spec->flags;
    d->latent_c = spec->latent_channels;
    d->groups = spec->groups;
    d->eps = spec->eps;
    d->layers.assign(spec->layers, spec->layers + spec->n_layers);
    d->ptrs.assign(params, params + need);
    d->packed.assign(need, nullptr);
    *out = d;
    return VAE_OK;
}

VAE_API void vae_decoder_destroy(vae_decoder_t* dec) {
    if (!dec) return;
    for (hipEvent_t e : dec->events) (void)hipEventDestroy(e);
    delete dec;
}

VAE_API vae_status_t vae_decoder_packed_weight_size(const vae_decoder_t* dec, size_t* bytes) {
    clear_error();
    if (!dec || !bytes) return fail(VAE_ERR_INVALID_ARG, "NULL argument");
    size_t total = 0;
    for_each_conv(*dec, [&](size_t, int32_t cin, int32_t cout, bool) {
        if (packable(*dec, cin, cout)) total += align_up((size_t)packed_weight_elems(cout, cin) * 2, 256);
    });
    *bytes = total;
    return VAE_OK;
}

VAE_API vae_status_t vae_decoder_pack_weights(vae_decoder_t* dec, void* buf, size_t bytes,
                                              vae_stream_t stream) {
    clear_error();
    if (!dec) return fail(VAE_ERR_INVALID_ARG, "decoder is NULL");
    size_t need = 0;
    VAE_TRY(vae_decoder_packed_weight_size(dec, &need));
    if (need > 0 && (!buf || bytes < need))
        return fail(VAE_ERR_WORKSPACE, "packed weight buffer too small", -1, (int64_t)bytes, -1,
                    (int64_t)need);
    if (reinterpret_cast<uintptr_t>(buf) % 256 != 0)
        return fail(VAE_ERR_INVALID_ARG, "packed weight buffer must be 256-byte aligned");
    uint8_t* out = static_cast<uint8_t*>(buf);
    vae_status_t st = VAE_OK;
    std::vector<const void*> packed(dec->ptrs.size(), nullptr);
    int conv_index = 0, bad = -1;
    for_each_conv(*dec, [&](size_t wi, int32_t cin, int32_t cout, bool f16) {
        if (st == VAE_OK && packable(*dec, cin, cout)) {
            st = launch_pack_weights(dec->ptrs[wi], cout, cin, out, as_stream(stream), f16);
            if (st != VAE_OK) bad = conv_index;
            packed[wi] = out;
            out += align_up((size_t)packed_weight_elems(cout, cin) * 2, 256);
        }
        ++conv_index;
    });
    if (st != VAE_OK) {
        if (st == VAE_ERR_UNSUPPORTED)   // a weight outside the fp16 range: name the conv
            return fail(st, "conv " + std::to_string(bad) + " (plan order): " + vae_last_error(),
                        -1, bad);
        return st;
    }
    dec->packed = packed;
    return VAE_OK;
}

VAE_API vae_status_t vae_decode_workspace_size(const vae_decoder_t* dec,
                                               const vae_tiling_desc_t* desc, size_t* bytes) {
    clear_error();
    if (!dec || !desc || !bytes) return fail(VAE_ERR_INVALID_ARG, "NULL argument");
    Layout L;
    std::vector<vae_tile_t> tiles;
    VAE_TRY(size_for(*dec, *desc, &L, &tiles));
    *bytes = L.total;
    return VAE_OK;
}

VAE_API vae_status_t vae_decode_tiled(const vae_decoder_t* dec_c, const vae_tensor_t* latent,
                                      const vae_tiling_desc_t* desc, vae_tensor_t* out, void* ws,
                                      size_t ws_bytes, vae_stream_t stream) {
    clear_error();
    vae_decoder* dec = const_cast<vae_decoder*>(dec_c);
    if (!dec || !desc) return fail(VAE_ERR_INVALID_ARG, "NULL decoder or tiling");
    VAE_TRY(check_tensor(latent, "latent"));
    VAE_TRY(check_tensor(out, "out"));
    if (latent->dtype != dec->dtype || latent->c != dec->latent_c)
        return fail(VAE_ERR_INVALID_ARG, "latent dtype/channels do not match the plan");
    if (latent->n != desc->n || latent->t != desc->t || latent->h != desc->h ||
        latent->w != desc->w)
        return fail(VAE_ERR_INVALID_ARG, "latent extents do not match the tiling desc");
    Layout L;
    std::vector<vae_tile_t> tiles;
    VAE_TRY(size_for(*dec, *desc, &L, &tiles));
    Shape os;
    int st, sh, sw;
    plan_output(*dec, *desc, &os, &st, &sh, &sw);
    if (out->dtype != VAE_DTYPE_F32 || out->n != os.n || out->t != os.t || out->h != os.h ||
        out->w != os.w || out->c != os.c)
        return fail(VAE_ERR_INVALID_ARG, "out must be fp32 of the decoded shape");
    if (!ws || ws_bytes < L.total)
        return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)ws_bytes, -1,
                    (int64_t)L.total);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(VAE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (overlaps(*latent, *out)) return fail(VAE_ERR_INVALID_ARG, "out overlaps latent");
    {
        const uint8_t* w0 = static_cast<const uint8_t*>(ws);
        vae_tensor_t wt{const_cast<uint8_t*>(w0), VAE_DTYPE_F32, 0, 1, 1, 1, 1,
                        (int64_t)(L.total / 4)};
        if (overlaps(wt, *latent) || overlaps(wt, *out))
            return fail(VAE_ERR_INVALID_ARG, "workspace overlaps latent or out");
    }

    dec->recs.clear();
    Runner r{dec, as_stream(stream), static_cast<uint8_t*>(ws), L, -1, 0};
    // clear the status word with a kernel (no memset node, so a captured decode replays right)
    VAE_TRY(launch_zero(r.ws + L.status, 16, r.s));
    VAE_TRY(r.mark(VAE_KIND_OTHER, -1, 0, 0));
    if (desc->mode == VAE_TILING_PATCH_HALO) {
        std::vector<Box> boxes;
        for (const vae_tile_t& t : tiles)
            boxes.push_back(Box{t.latent.t0, t.latent.t1, t.latent.h0, t.latent.h1, t.latent.w0,
                                t.latent.w1});
        r.per_patch = dec->launch == VAE_LAUNCH_PER_PATCH && boxes.size() > 1;
        if (!clipped(*dec, *desc)) {
            VAE_TRY(r.run(*latent, boxes, *out));
            return VAE_OK;
        }
        // clip by clip: clip c decodes latent frames [c0, c0 + n) into output frames
        // [o0, o1), each conv carrying its last two input frames into the next clip
        if (latent->n != 1)
            return fail(VAE_ERR_UNSUPPORTED, "a clip-by-clip decode takes one sample");
        const int64_t R = desc->scale_t;
        const int64_t lf = Shape{latent->n, 1, latent->h, latent->w, latent->c,
                                 latent->dtype}.frame_bytes();
        const int64_t of = Shape{out->n, 1, out->h, out->w, out->c, out->dtype}.frame_bytes();
        r.clips = true;
        for (int64_t c0 = 0, c = 0; c0 < latent->t; c0 += dec->clip, ++c) {
            const int64_t n = std::min<int64_t>(dec->clip, latent->t - c0);
            const int64_t o0 = c0 == 0 ? 0 : (c0 - 1) * R + 1, o1 = (c0 + n - 1) * R + 1;
            vae_tensor_t lc = *latent, oc = *out;
            lc.data = static_cast<uint8_t*>(latent->data) + c0 * lf;
            lc.t = n;
            oc.data = static_cast<uint8_t*>(out->data) + o0 * of;
            oc.t = o1 - o0;
            r.first_clip = c0 == 0;
            r.tile = (int32_t)c;
            VAE_TRY(r.run(lc, boxes, oc));
        }
    } else {
        AxisTiling ax[3];
        overlap_axes(*desc, ax);
        for (size_t i = 0; i < tiles.size(); ++i) {
            const vae_tile_t& t = tiles[i];
            r.tile = (int32_t)i;
            const Box lb{t.latent.t0, t.latent.t1, t.latent.h0, t.latent.h1, t.latent.w0,
                         t.latent.w1};
            Shape cs{latent->n, lb.bt(), lb.bh(), lb.bw(), latent->c, latent->dtype};
            vae_tensor_t crop = tensor_of(r.ws + L.crop, cs);
            VAE_TRY(launch_crop(*latent, lb, crop, r.s));
            VAE_TRY(r.mark(VAE_KIND_OTHER, -1, 0, 2.0 * (double)cs.bytes()));
            std::vector<Box> one{Box{0, (int32_t)cs.t, 0, (int32_t)cs.h, 0, (int32_t)cs.w}};
            Shape ts{os.n, t.out.t1 - t.out.t0, t.out.h1 - t.out.h0, t.out.w1 - t.out.w0, os.c,
                     VAE_DTYPE_F32};
            vae_tensor_t tile_out = tensor_of(r.ws + L.tile, ts);
            VAE_TRY(r.run(crop, one, tile_out));
            const Box ob{t.out.t0, t.out.t1, t.out.h0, t.out.h1, t.out.w0, t.out.w1};
            if (i == 0) VAE_TRY(launch_zero(out->data, numel(*out) * 4, r.s));
            VAE_TRY(launch_merge(tile_out, ob, MergeRamps{t}, *out, r.s));
            double mb = 3.0 * (double)ts.bytes() + (i == 0 ? (double)numel(*out) * 4 : 0.0);
            if (i + 1 == tiles.size()) {
                VAE_TRY(launch_merge_finalize(*out, ax[0], ax[1], ax[2], r.s));
                mb += 2.0 * (double)numel(*out) * 4;
            }
            VAE_TRY(r.mark(VAE_KIND_MERGE, -1, 0, mb));
        }
    }
    return VAE_OK;
}

VAE_API vae_status_t vae_decoder_set_launch(vae_decoder_t* dec, int32_t launch) {
    clear_error();
    if (!dec) return fail(VAE_ERR_INVALID_ARG, "decoder is NULL");
    if (launch != VAE_LAUNCH_MERGED && launch != VAE_LAUNCH_PER_PATCH)
        return fail(VAE_ERR_INVALID_ARG, "launch must be VAE_LAUNCH_MERGED or VAE_LAUNCH_PER_PATCH");
    dec->launch = launch;
    return VAE_OK;
}

VAE_API vae_status_t vae_decoder_set_clip_frames(vae_decoder_t* dec, int32_t frames) {
    clear_error();
    if (!dec) return fail(VAE_ERR_INVALID_ARG, "decoder is NULL");
    if (frames < 0) return fail(VAE_ERR_INVALID_ARG, "clip frames must be >= 0", -1, frames);
    if (frames > 0) {
        if (dec->dtype != VAE_DTYPE_BF16)
            return fail(VAE_ERR_UNSUPPORTED, "a clip-by-clip decode needs a bf16 plan");
        for (const vae_layer_desc_t& l : dec->layers)
            if (l.op != VAE_OP_CONV && l.op != VAE_OP_RES_RMS && l.op != VAE_OP_RMS_SILU &&
                l.op != VAE_OP_ATTN && l.op != VAE_OP_D2S && l.op != VAE_OP_NEAREST)
                return fail(VAE_ERR_UNSUPPORTED,
                            "a clip-by-clip decode takes convs, RMS norms, frame attention and "
                            "upsamplings only (GroupNorm statistics span every frame)");
    }
    dec->clip = frames;
    return VAE_OK;
}

VAE_API vae_status_t vae_decode_status(const vae_decoder_t* dec, const vae_tiling_desc_t* desc,
                                       const void* ws, size_t ws_bytes, int32_t* flags,
                                       vae_stream_t stream) {
    clear_error();
    if (!dec || !desc || !ws || !flags) return fail(VAE_ERR_INVALID_ARG, "NULL argument");
    Layout L;
    std::vector<vae_tile_t> tiles;
    VAE_TRY(size_for(*dec, *desc, &L, &tiles));
    if (ws_bytes < L.total)
        return fail(VAE_ERR_WORKSPACE, "workspace too small", -1, (int64_t)ws_bytes, -1,
                    (int64_t)L.total);
    uint32_t word = 0;
    VAE_HIP_CHECK(hipStreamSynchronize(as_stream(stream)));
    VAE_HIP_CHECK(hipMemcpy(&word, static_cast<const uint8_t*>(ws) + L.status, sizeof(word),
                            hipMemcpyDeviceToHost));
    *flags = (int32_t)(word ? VAE_STATUS_NONFINITE : 0);
    return VAE_OK;
}

VAE_API vae_status_t vae_decoder_set_timing(vae_decoder_t* dec, int32_t enable) {
    clear_error();
    if (!dec) return fail(VAE_ERR_INVALID_ARG, "decoder is NULL");
    dec->timing = enable != 0;
    dec->recs.clear();
    return VAE_OK;
}

VAE_API vae_status_t vae_decoder_get_timing(vae_decoder_t* dec, vae_op_timing_t* out,
                                            int32_t capacity, int32_t* n) {
    clear_error();
    if (!dec || !n) return fail(VAE_ERR_INVALID_ARG, "NULL argument");
    *n = (int32_t)dec->recs.size();
    if (!out || dec->recs.empty()) return VAE_OK;
    if (capacity < *n) return fail(VAE_ERR_INVALID_ARG, "capacity too small", -1, capacity, -1, *n);
    VAE_HIP_CHECK(hipEventSynchronize(dec->events[dec->recs.size()]));
    for (size_t i = 0; i < dec->recs.size(); ++i) {
        float ms = 0.0f;
        VAE_HIP_CHECK(hipEventElapsedTime(&ms, dec->events[i], dec->events[i + 1]));
        const auto& r = dec->recs[i];
        out[i] = vae_op_timing_t{r.kind, r.layer, r.tile, 0, (double)ms, r.flops, r.bytes};
    }
    return VAE_OK;
}

}  // extern "C"
