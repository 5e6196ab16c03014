// C-ABI entry points (declared in include/deltalog.h): descriptor checks,
// state-block layout, argument validation and kernel dispatch.  No C++
// exception crosses this boundary; every failure is a dl_status plus a
// thread-local message.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include <algorithm>

#include "dl_common.hpp"

struct dl_state {
    dl_desc desc;
    dl::Params p;
    void *mem;
    size_t bytes;
    hipEvent_t ev_start, ev_stop;   // armed by dl_time_next_launch, consumed by one launch
};

namespace {

thread_local char g_err[512];

dl_status fail(dl_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dl_status ok() {
    g_err[0] = '\0';
    return DL_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
    size_t off_flags, off_fill, off_base, off_k, off_v, off_g, off_b, off_t;
    size_t off_codes, off_scale, off_kept, off_kidx, total;
};

dl_status check_desc(const dl_desc *d) {
    if (!d)
        return fail(DL_ERR_INVALID, "descriptor is NULL");
    if (d->variant < DL_GDN || d->variant > DL_GDN2)
        return fail(DL_ERR_INVALID, "unknown variant %d", d->variant);
    if (d->units < 1 || d->heads < 1)
        return fail(DL_ERR_INVALID, "units (%d) and heads (%d) must be >= 1", d->units, d->heads);
    if (d->in_dtype != DL_F32 && d->in_dtype != DL_BF16)
        return fail(DL_ERR_INVALID, "unknown input dtype %d", d->in_dtype);
    if (d->log_len < 0)
        return fail(DL_ERR_INVALID, "log_len must be >= 0, got %d", d->log_len);
    if (d->merge_on_step != 0 && d->merge_on_step != 1)
        return fail(DL_ERR_INVALID, "merge_on_step must be 0 or 1, got %d", d->merge_on_step);
    if (d->log_form != DL_LOG_WY && d->log_form != DL_LOG_FACTORS)
        return fail(DL_ERR_INVALID, "unknown log_form %d", d->log_form);
    if (d->d_k != d->d_v)
        return fail(DL_ERR_UNSUPPORTED, "d_k (%d) != d_v (%d) is not built", d->d_k, d->d_v);
    if (d->d_k != 64 && d->d_k != 128)
        return fail(DL_ERR_UNSUPPORTED, "d = %d is not built (64 or 128)", d->d_k);
    if (d->log_len > 64)
        return fail(DL_ERR_UNSUPPORTED, "log_len %d > 64 is not built", d->log_len);
    if (d->variant == DL_GDN2 && d->log_len > 0 && d->log_form != DL_LOG_FACTORS)
        return fail(DL_ERR_UNSUPPORTED, "the gated variant's log is built in the factor form only");
    if (d->base_format != DL_BASE_F32 && d->base_format != DL_BASE_I8)
        return fail(DL_ERR_INVALID, "unknown base format %d", d->base_format);
    if (d->base_format == DL_BASE_F32 && d->kept_channels != 0)
        return fail(DL_ERR_INVALID, "kept_channels applies to an INT8 base only");
    if (d->base_format == DL_BASE_I8) {
        if (d->kept_channels < 0 || d->kept_channels > 16)
            return fail(DL_ERR_INVALID, "kept_channels must be 0 .. 16, got %d", d->kept_channels);
        if (d->log_len < 1 || d->log_form != DL_LOG_FACTORS || d->variant == DL_RWKV6)
            return fail(DL_ERR_UNSUPPORTED,
                        "an INT8 base is built for factor-form logs of the delta-rule variants");
    }
    const size_t pairs = (size_t)d->units * (size_t)d->heads;
    if (pairs > (size_t)0x7fffffff)
        return fail(DL_ERR_INVALID, "units * heads too large");
    return DL_OK;
}

// The additive-factor log applies to the delta-rule variants; RWKV6's log
// has that form already.
bool factors_form(const dl_desc &d) { return d.log_form == DL_LOG_FACTORS && d.variant != DL_RWKV6; }

Layout layout_of(const dl_desc &d) {
    Layout l;
    const size_t pairs = (size_t)d.units * d.heads;
    const size_t es = d.in_dtype == DL_BF16 ? 2 : 4;
    const size_t L = d.log_len;
    const size_t gch = d.variant == DL_GDN ? 1 : d.d_k;
    const bool af = factors_form(d);
    size_t off = 0;
    l.off_flags = off;
    off = align256(off + 256);
    l.off_fill = off;
    off = align256(off + pairs * 4);
    const bool q8 = d.base_format == DL_BASE_I8;
    const size_t M = q8 ? d.kept_channels : 0;
    l.off_base = off;
    off = align256(off + (q8 ? 0 : pairs * d.d_v * d.d_k * 4));
    l.off_codes = off;
    off = align256(off + (q8 ? pairs * d.d_v * d.d_k : 0));
    l.off_scale = off;
    off = align256(off + (q8 ? pairs * d.d_v * 4 : 0));
    l.off_kept = off;
    off = align256(off + pairs * d.d_v * M * 4);
    l.off_kidx = off;
    off = align256(off + (size_t)d.heads * M * 4);
    l.off_k = off;
    off = align256(off + pairs * L * d.d_k * es);
    l.off_v = off;
    off = align256(off + pairs * L * d.d_v * (af ? 4 : es));
    l.off_g = off;
    off = align256(off + pairs * L * gch * 4);
    l.off_b = off;
    off = align256(off + ((d.variant == DL_RWKV6 || af) ? 0 : pairs * L * 4));
    l.off_t = off;
    off = align256(off + (af ? 0 : pairs * (size_t)dl::packed_t_len(d.variant, d.log_len) * 4));
    l.total = off;
    return l;
}

// Stream the state (nontemporal loads and stores) when what the steps re-read
// does not fit MI355X's 256 MiB Infinity Cache.  Eager: the state itself.
// With a log, every step reads the whole base and the logged entries; once
// base and log together are well past the cache (1.5x), streaming the base
// keeps the log entries, read back by every step, resident instead of
// letting both thrash.  The base is everything from the fp32 base (or the
// INT8 codes, scales and kept channels) up to the log, the log everything
// after it.
bool streams(const dl_desc &d, const Layout &l) {
    const size_t base_bytes = l.off_k - l.off_base;
    const size_t log_bytes = l.total - l.off_k;
    return d.log_len == 0 ? base_bytes > ((size_t)256 << 20)
                          : base_bytes + log_bytes > ((size_t)384 << 20);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dl_status check_rows(const dl_state *st, int32_t rows, const int32_t *slot_idx) {
    if (!st)
        return fail(DL_ERR_INVALID, "state handle is NULL");
    if (rows < 0)
        return fail(DL_ERR_INVALID, "rows must be >= 0, got %d", rows);
    if (!slot_idx && rows > st->desc.units)
        return fail(DL_ERR_INVALID, "rows (%d) > units (%d) without slot_idx", rows, st->desc.units);
    if (slot_idx && !aligned(slot_idx, 4))
        return fail(DL_ERR_INVALID, "slot_idx must be 4-byte aligned");
    if ((size_t)rows * st->desc.heads > (size_t)0x7fffffff)
        return fail(DL_ERR_INVALID, "rows * heads too large for one launch");
    return DL_OK;
}

dl_status check_step_args(const dl_state *st, int32_t rows, const int32_t *slot_idx,
                          const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *o) {
    dl_status s = check_rows(st, rows, slot_idx);
    if (s != DL_OK)
        return s;
    if (!q || !k || !v || !g || !o)
        return fail(DL_ERR_INVALID, "q, k, v, g and o must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(DL_ERR_INVALID, "q, k, v and o must be 16-byte aligned");
    if (!aligned(g, st->desc.variant == DL_GDN ? 4 : 16))
        return fail(DL_ERR_INVALID, "g must be %d-byte aligned",
                    st->desc.variant == DL_GDN ? 4 : 16);
    if (st->desc.variant != DL_RWKV6) {
        if (!beta)
            return fail(DL_ERR_INVALID, "beta is required for the delta-rule variants");
        const int ba = st->desc.variant == DL_GDN2 ? 16 : 4;
        if (!aligned(beta, ba))
            return fail(DL_ERR_INVALID, "beta must be %d-byte aligned", ba);
    }
    return DL_OK;
}

// The step/readout kernels stage the key side of the log (keys, decays,
// betas, key-side factors) in LDS; the request must fit the current
// device's per-workgroup LDS (160 KiB on gfx950).
dl_status check_lds(const dl_state *st) {
    const int es = st->desc.in_dtype == DL_BF16 ? 2 : 4;
    const dl::StepPlan lp = dl::step_plan(st->desc.variant, st->desc.d_k, es, st->desc.log_len,
                                          st->desc.merge_on_step != 0);
    const int bytes = st->p.af ? dl::af_plan(st->desc.d_k, st->desc.log_len, true).bytes : lp.bytes;
    if (bytes <= 65536)
        return DL_OK;
    int dev = 0, max_lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return fail(DL_ERR_LAUNCH, "cannot query the device's LDS size");
    if (bytes > max_lds)
        return fail(DL_ERR_UNSUPPORTED, "log of %d entries needs %d bytes of LDS (device limit %d)",
                    st->desc.log_len, bytes, max_lds);
    return DL_OK;
}

dl::Launch launch_of(const dl_state *st, void *stream) {
    return dl::Launch{static_cast<hipStream_t>(stream), st->ev_start, st->ev_stop};
}

// The block's parameters for one step launch over `rows` rows, taken in
// `row_order` (NULL: input order).
dl::Params with_rows(const dl::Params &base, int32_t rows, const int32_t *row_order) {
    dl::Params p = base;
    p.rows = rows;
    p.row_order = row_order;
    return p;
}

// Result of one launch; a launch consumes the events dl_time_next_launch armed.
dl_status launched(dl_state *st, hipError_t e, const char *what) {
    st->ev_start = nullptr;
    st->ev_stop = nullptr;
    if (e != hipSuccess)
        return fail(DL_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

size_t dl_state_bytes(const dl_desc *desc) {
    if (check_desc(desc) != DL_OK)
        return 0;
    return layout_of(*desc).total;
}

dl_status dl_state_alloc(const dl_desc *desc, void *dev_mem, size_t bytes, void *stream,
                         dl_state **out) {
    dl_status s = check_desc(desc);
    if (s != DL_OK)
        return s;
    if (!out)
        return fail(DL_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (!dev_mem)
        return fail(DL_ERR_INVALID, "device memory is NULL");
    if (!aligned(dev_mem, 256))
        return fail(DL_ERR_INVALID, "device memory must be 256-byte aligned");
    const Layout l = layout_of(*desc);
    if (bytes < l.total)
        return fail(DL_ERR_SIZE, "state block needs %zu bytes, got %zu", l.total, bytes);
    dl_state *st = new (std::nothrow) dl_state;
    if (!st)
        return fail(DL_ERR_INVALID, "out of host memory");
    st->desc = *desc;
    st->ev_start = nullptr;
    st->ev_stop = nullptr;
    st->mem = dev_mem;
    st->bytes = bytes;
    char *m = static_cast<char *>(dev_mem);
    dl::Params &p = st->p;
    p.variant = desc->variant;
    p.units = desc->units;
    p.heads = desc->heads;
    p.D = desc->d_k;
    p.L = desc->log_len;
    p.dtype = desc->in_dtype;
    p.flags = reinterpret_cast<int *>(m + l.off_flags);
    p.fuse = desc->merge_on_step;
    p.rows = 0;
    p.row_order = nullptr;
    p.af = factors_form(*desc) ? 1 : 0;
    p.stream = streams(*desc, l);
    p.fill = reinterpret_cast<int *>(m + l.off_fill);
    p.q8 = desc->base_format == DL_BASE_I8 ? 1 : 0;
    p.M = p.q8 ? desc->kept_channels : 0;
    p.base = p.q8 ? nullptr : reinterpret_cast<float *>(m + l.off_base);
    p.codes = p.q8 ? reinterpret_cast<int8_t *>(m + l.off_codes) : nullptr;
    p.scale = p.q8 ? reinterpret_cast<float *>(m + l.off_scale) : nullptr;
    p.kept = p.q8 ? reinterpret_cast<float *>(m + l.off_kept) : nullptr;
    p.kidx = p.q8 ? reinterpret_cast<int *>(m + l.off_kidx) : nullptr;
    const bool has_log = desc->log_len > 0;
    p.log_k = has_log ? m + l.off_k : nullptr;
    p.log_v = has_log ? m + l.off_v : nullptr;
    p.log_g = has_log ? reinterpret_cast<float *>(m + l.off_g) : nullptr;
    p.log_beta = (has_log && desc->variant != DL_RWKV6 && !p.af)
                     ? reinterpret_cast<float *>(m + l.off_b)
                     : nullptr;
    p.log_t = (!p.af && dl::packed_t_len(desc->variant, desc->log_len) > 0)
                  ? reinterpret_cast<float *>(m + l.off_t)
                  : nullptr;
    hipError_t e = dl::launch_zero(dev_mem, l.total,
                                   dl::Launch{static_cast<hipStream_t>(stream), nullptr, nullptr});
    if (e == hipSuccess)
        e = dl::launch_kept_default(p, dl::Launch{static_cast<hipStream_t>(stream), nullptr, nullptr});
    if (e != hipSuccess) {
        delete st;
        return fail(DL_ERR_LAUNCH, "zeroing the state block: %s", hipGetErrorString(e));
    }
    *out = st;
    return ok();
}

dl_status dl_state_free(dl_state *st) {
    delete st;
    return ok();
}

dl_status dl_state_view(const dl_state *st, dl_state_ptrs *out) {
    if (!st || !out)
        return fail(DL_ERR_INVALID, "state and out must be non-NULL");
    out->base = st->p.base;
    out->log_k = st->p.log_k;
    out->log_v = st->p.log_v;
    out->log_g = st->p.log_g;
    out->log_beta = st->p.log_beta;
    out->log_t = st->p.log_t;
    out->fill = st->p.fill;
    out->flags = st->p.flags;
    out->base_codes = st->p.codes;
    out->base_scale = st->p.scale;
    out->base_kept = st->p.kept;
    out->kept_idx = st->p.kidx;
    return ok();
}

dl_status dl_decode_step_eager_ordered(dl_state *st, int32_t rows, const int32_t *slot_idx,
                                       const int32_t *row_order, const void *q, const void *k,
                                       const void *v, const float *g, const float *beta, float *o,
                                       void *stream) {
    dl_status s = check_step_args(st, rows, slot_idx, q, k, v, g, beta, o);
    if (s != DL_OK)
        return s;
    if (row_order && !aligned(row_order, 4))
        return fail(DL_ERR_INVALID, "row_order must be 4-byte aligned");
    if (st->p.q8)
        return fail(DL_ERR_UNSUPPORTED, "the eager step is built for an fp32 state only");
    if (rows == 0)
        return ok();
    const dl::Params p = with_rows(st->p, rows, row_order);
    return launched(st, dl::launch_eager(p, rows, slot_idx, q, k, v, g, beta, o, launch_of(st, stream)),
                    "eager step launch");
}

dl_status dl_decode_step_eager(dl_state *st, int32_t rows, const int32_t *slot_idx,
                               const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *o, void *stream) {
    return dl_decode_step_eager_ordered(st, rows, slot_idx, nullptr, q, k, v, g, beta, o, stream);
}

dl_status dl_decode_step_log_ordered(dl_state *st, int32_t rows, const int32_t *slot_idx,
                                     const int32_t *row_order, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta, float *o,
                                     void *stream) {
    dl_status s = check_step_args(st, rows, slot_idx, q, k, v, g, beta, o);
    if (s != DL_OK)
        return s;
    if (row_order && !aligned(row_order, 4))
        return fail(DL_ERR_INVALID, "row_order must be 4-byte aligned");
    if (st->desc.log_len < 1)
        return fail(DL_ERR_INVALID, "this state has no log (log_len = 0)");
    s = check_lds(st);
    if (s != DL_OK)
        return s;
    if (rows == 0)
        return ok();
    const dl::Launch ln = launch_of(st, stream);
    const dl::Params p = with_rows(st->p, rows, row_order);
    return launched(st,
                    p.af ? dl::launch_af_step(p, rows, slot_idx, q, k, v, g, beta, o, ln)
                         : dl::launch_log_step(p, rows, slot_idx, q, k, v, g, beta, o, ln),
                    "log step launch");
}

dl_status dl_decode_step_log(dl_state *st, int32_t rows, const int32_t *slot_idx,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *o, void *stream) {
    return dl_decode_step_log_ordered(st, rows, slot_idx, nullptr, q, k, v, g, beta, o, stream);
}

static dl_status merge_common(dl_state *st, int32_t rows, const int32_t *slot_idx, int32_t mode,
                              void *stream, bool wy) {
    dl_status s = check_rows(st, rows, slot_idx);
    if (s != DL_OK)
        return s;
    if (mode != DL_MERGE_FULL && mode != DL_MERGE_ALL)
        return fail(DL_ERR_INVALID, "unknown merge mode %d", mode);
    if (st->desc.log_len < 1 || rows == 0)
        return ok();
    const dl::Launch ln = launch_of(st, stream);
    const hipError_t e = st->p.af ? dl::launch_af_merge(st->p, rows, slot_idx, mode, ln)
                         : wy     ? dl::launch_merge_wy(st->p, rows, slot_idx, mode, ln)
                                  : dl::launch_merge_replay(st->p, rows, slot_idx, mode, ln);
    return launched(st, e, "merge launch");
}

dl_status dl_merge(dl_state *st, int32_t rows, const int32_t *slot_idx, int32_t mode,
                   void *stream) {
    return merge_common(st, rows, slot_idx, mode, stream, true);
}

dl_status dl_merge_replay(dl_state *st, int32_t rows, const int32_t *slot_idx, int32_t mode,
                          void *stream) {
    return merge_common(st, rows, slot_idx, mode, stream, false);
}

static dl_status base_io(dl_state *st, int32_t rows, const int32_t *slot_idx, const void *buf,
                         void *stream, bool import) {
    dl_status s = check_rows(st, rows, slot_idx);
    if (s != DL_OK)
        return s;
    if (!buf || !aligned(buf, 16))
        return fail(DL_ERR_INVALID, "the state buffer must be non-NULL and 16-byte aligned");
    if (rows == 0)
        return ok();
    const dl::Launch ln = launch_of(st, stream);
    const hipError_t e =
        import ? dl::launch_base_import(st->p, rows, slot_idx, static_cast<const float *>(buf), ln)
               : dl::launch_base_export(st->p, rows, slot_idx, static_cast<float *>(const_cast<void *>(buf)),
                                        ln);
    return launched(st, e, import ? "base import launch" : "base export launch");
}

dl_status dl_base_import(dl_state *st, int32_t rows, const int32_t *slot_idx, const float *src,
                         void *stream) {
    return base_io(st, rows, slot_idx, src, stream, true);
}

dl_status dl_base_export(dl_state *st, int32_t rows, const int32_t *slot_idx, float *dst,
                         void *stream) {
    return base_io(st, rows, slot_idx, dst, stream, false);
}

dl_status dl_readout(dl_state *st, int32_t rows, const int32_t *slot_idx, const void *q,
                     float *o, void *stream) {
    dl_status s = check_rows(st, rows, slot_idx);
    if (s != DL_OK)
        return s;
    if (!q || !o)
        return fail(DL_ERR_INVALID, "q and o must be non-NULL");
    if (!aligned(q, 16) || !aligned(o, 16))
        return fail(DL_ERR_INVALID, "q and o must be 16-byte aligned");
    s = check_lds(st);
    if (s != DL_OK)
        return s;
    if (rows == 0)
        return ok();
    const dl::Launch ln = launch_of(st, stream);
    return launched(st,
                    st->p.af ? dl::launch_af_readout(st->p, rows, slot_idx, q, o, ln)
                             : dl::launch_readout(st->p, rows, slot_idx, q, o, ln),
                    "readout launch");
}

dl_status dl_state_check(dl_state *st, void *stream, int32_t *flags_out) {
    if (!st)
        return fail(DL_ERR_INVALID, "state handle is NULL");
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t h = 0;
    hipError_t e = hipMemcpyAsync(&h, st->p.flags, sizeof(int32_t), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess)
        e = hipStreamSynchronize(hs);
    if (e != hipSuccess)
        return fail(DL_ERR_LAUNCH, "reading device flags: %s", hipGetErrorString(e));
    if (flags_out)
        *flags_out = h;
    if (h != 0) {
        e = dl::launch_zero(st->p.flags, 256, dl::Launch{hs, nullptr, nullptr});
        if (e != hipSuccess)
            return fail(DL_ERR_LAUNCH, "clearing device flags: %s", hipGetErrorString(e));
        return fail(DL_ERR_STATE,
                    "device flags 0x%x (1: log full, 2: eager on non-empty log, 4: bad slot, "
                    "8: bad kept channels)", h);
    }
    return ok();
}

dl_status dl_time_next_launch(dl_state *st, void *start_event, void *stop_event) {
    if (!st)
        return fail(DL_ERR_INVALID, "state handle is NULL");
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(DL_ERR_INVALID, "give both events or neither");
    st->ev_start = static_cast<hipEvent_t>(start_event);
    st->ev_stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

const char *dl_last_error(void) { return g_err; }

int32_t dl_version(void) { return 100; }

dl_status dl_suggest_log_len(const dl_desc *desc, int32_t *L_out, double *bytes_out) {
    if (!desc || !L_out)
        return fail(DL_ERR_INVALID, "desc and L_out must be non-NULL");
    dl_desc d = *desc;
    d.log_len = 1;
    const dl_status cs = check_desc(&d);
    if (cs != DL_OK)
        return cs;
    const double es = d.in_dtype == DL_BF16 ? 2.0 : 4.0;
    const double dk = d.d_k, dv = d.d_v;
    // the base a step reads and a merge writes: fp32, or INT8 codes, row
    // scales and the kept channels
    const double St = d.base_format == DL_BASE_I8 ? dv * dk + 4.0 * dv * (1.0 + d.kept_channels)
                                                  : 4.0 * dv * dk;
    const bool af = factors_form(d);
    const double gb = d.variant == DL_GDN ? 4.0 : 4.0 * dk;       // decay bytes per entry
    const double bb = d.variant == DL_RWKV6 ? 0.0                 // beta bytes per input
                      : d.variant == DL_GDN2 ? 4.0 * (dk + dv) : 4.0;
    const double In = (2.0 * dk + dv) * es + gb + bb;
    const double Out = 4.0 * dv;
    // logged entry: key, value (fp32 factor under the additive-factor form), decay, beta
    const double E = dk * es + dv * (af ? 4.0 : es) + gb + (af ? 0.0 : bb);
    const bool delta = d.variant != DL_RWKV6 && !af;             // R columns are logged
    const bool fuse = d.merge_on_step != 0;
    int best = 1;
    double best_cost = 0.0, best_bytes = 0.0;
    for (int L = 1; L <= 64; ++L) {
        const double c = (L - 1) / 2.0;                           // mean logged entries read
        const double rt = delta ? 4.0 * ((L - 1.0) * (L - 2.0) / 6.0 + c) : 0.0;
        double bytes = St + c * E + E + In + Out + 8.0 + rt;
        // merging in place writes the base once per L steps and saves that
        // step's append; a separate merge reads and writes the base and reads the log
        bytes += fuse ? (St - E) / L : (2.0 * St + L * E + 8.0) / L;
        const bool chunked = !af && d.variant == DL_KDA && d.d_k == 128 && L > 32 && !fuse;
        const int lds = af        ? dl::af_plan(d.d_k, L, fuse).bytes
                        : chunked ? dl::chunk_plan(d.d_k, (int)es, L).bytes
                                  : dl::step_plan(d.variant, d.d_k, (int)es, L, fuse).bytes;
        const int wgs = std::min(4, (160 * 1024) / std::max(lds, 1));
        const double cost = bytes * 4.0 / std::max(wgs, 1);
        if (L == 1 || cost < best_cost) {
            best = L;
            best_cost = cost;
            best_bytes = bytes;
        }
    }
    *L_out = best;
    if (bytes_out)
        *bytes_out = best_bytes;
    return ok();
}

dl_status dl_state_streams(const dl_desc *desc, int32_t *streams_out) {
    if (!streams_out)
        return fail(DL_ERR_INVALID, "streams_out must be non-NULL");
    const dl_status cs = check_desc(desc);
    if (cs != DL_OK)
        return cs;
    *streams_out = streams(*desc, layout_of(*desc)) ? 1 : 0;
    return ok();
}

dl_status dl_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes, void *stream,
                          void *start_event, void *stop_event) {
    if (mode != DL_PROBE_READ && mode != DL_PROBE_COPY)
        return fail(DL_ERR_INVALID, "unknown probe mode %d", mode);
    if (!src || !dst)
        return fail(DL_ERR_INVALID, "src and dst must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
        return fail(DL_ERR_INVALID, "src and dst must be 16-byte aligned");
    if (bytes == 0 || bytes % 16 != 0)
        return fail(DL_ERR_INVALID, "bytes must be a positive multiple of 16, got %zu", bytes);
    if (dl::probe_read_outputs(bytes) > 0x7fffffffu)
        return fail(DL_ERR_UNSUPPORTED, "buffer of %zu bytes is too large for one launch", bytes);
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(DL_ERR_INVALID, "give both events or neither");
    const dl::Launch ln{static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                        static_cast<hipEvent_t>(stop_event)};
    const hipError_t e = dl::launch_stream_probe(mode, src, dst, bytes, ln);
    if (e != hipSuccess)
        return fail(DL_ERR_LAUNCH, "stream probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
