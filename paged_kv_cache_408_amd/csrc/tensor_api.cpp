// pa_kv_write_t and pa_decode_t: the two kernel calls over tensor views.  Host code only: every
// view is checked (dtype, rank, shape agreement, C-contiguity) before the plain entry point is
// called with the sizes the views carry, so a caller's shape mistake is reported here, by
// argument name, instead of becoming a wrong-sized launch.
#include <cstdint>

#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

const char* dtype_name(int dt) {
    switch (dt) {
        case PA_DTYPE_F32: return "f32";
        case PA_DTYPE_BF16: return "bf16";
        case PA_DTYPE_FP8_E4M3: return "fp8";
        case PA_DTYPE_MXFP4: return "mxfp4";
        case PA_DTYPE_I32: return "int32";
        case PA_DTYPE_I64: return "int64";
    }
    return "unknown";
}

// A view of rank `ndim` that is C-contiguous (all strides 0 for the packed MXFP4 cache).
int check_view(const pa_tensor* t, int ndim, const char* fn, const char* what) {
    if (!t) return fail(PA_ERR_INVALID, "%s: %s is NULL", fn, what);
    if (t->ndim != ndim) return fail(PA_ERR_INVALID, "%s: %s has %d dims, %d expected", fn, what, t->ndim, ndim);
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] < 0) return fail(PA_ERR_INVALID, "%s: %s shape[%d] = %lld", fn, what, i, (long long)t->shape[i]);
    if (t->dtype == PA_DTYPE_MXFP4) {
        for (int i = 0; i < ndim; ++i)
            if (t->stride[i] != 0)
                return fail(PA_ERR_INVALID, "%s: %s is an MXFP4 cache: give its strides as 0 (packed tiles)", fn, what);
        return PA_OK;
    }
    int64_t want = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        if (t->shape[i] > 1 && t->stride[i] != want)
            return fail(PA_ERR_INVALID, "%s: %s is not C-contiguous (stride[%d] = %lld, %lld expected)", fn, what, i,
                        (long long)t->stride[i], (long long)want);
        want *= t->shape[i];
    }
    return PA_OK;
}

int check_dtype(const pa_tensor* t, int dtype, const char* fn, const char* what) {
    if (t->dtype != dtype)
        return fail(PA_ERR_INVALID, "%s: %s is %s, %s expected", fn, what, dtype_name(t->dtype), dtype_name(dtype));
    return PA_OK;
}

bool same_shape(const pa_tensor* a, const pa_tensor* b) {
    if (a->ndim != b->ndim) return false;
    for (int i = 0; i < a->ndim; ++i)
        if (a->shape[i] != b->shape[i]) return false;
    return true;
}

int32_t narrow(int64_t x) { return x > 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(x); }

}  // namespace

extern "C" {

int pa_kv_write_t(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping, pa_tensor* k_cache,
                  pa_tensor* v_cache, const pa_opts* opts) {
    static const char* fn = "pa_kv_write_t";
    pagedkv::clear_error();
    const pa_opts none{};
    const pa_opts& o = opts ? *opts : none;
    if (int rc = check_view(k, 3, fn, "k")) return rc;
    if (int rc = check_view(v, 3, fn, "v")) return rc;
    if (int rc = check_view(slot_mapping, 1, fn, "slot_mapping")) return rc;
    if (int rc = check_view(k_cache, 4, fn, "k_cache")) return rc;
    if (int rc = check_view(v_cache, 4, fn, "v_cache")) return rc;
    if (int rc = check_dtype(slot_mapping, PA_DTYPE_I64, fn, "slot_mapping")) return rc;
    if (!same_shape(k, v) || k->dtype != v->dtype) return fail(PA_ERR_INVALID, "%s: k and v differ in shape or dtype", fn);
    if (!same_shape(k_cache, v_cache) || k_cache->dtype != v_cache->dtype)
        return fail(PA_ERR_INVALID, "%s: k_cache and v_cache differ in shape or dtype", fn);
    if (slot_mapping->shape[0] != k->shape[0])
        return fail(PA_ERR_INVALID, "%s: slot_mapping has %lld entries for %lld tokens", fn,
                    (long long)slot_mapping->shape[0], (long long)k->shape[0]);
    if (k_cache->shape[1] != k->shape[1] || k_cache->shape[3] != k->shape[2])
        return fail(PA_ERR_INVALID, "%s: k [%lld, %lld, %lld] does not match the cache's heads / head dim [%lld, %lld]", fn,
                    (long long)k->shape[0], (long long)k->shape[1], (long long)k->shape[2], (long long)k_cache->shape[1],
                    (long long)k_cache->shape[3]);
    if (k_cache->shape[1] > 0x7fffffff || k_cache->shape[2] > 0x7fffffff || k_cache->shape[3] > 0x7fffffff)
        return fail(PA_ERR_INVALID, "%s: cache dims beyond int32", fn);
    return pa_kv_write(k->data, v->data, static_cast<const int64_t*>(slot_mapping->data), k->shape[0], k_cache->data,
                       v_cache->data, k_cache->shape[0], static_cast<int32_t>(k_cache->shape[1]),
                       static_cast<int32_t>(k_cache->shape[3]), static_cast<int32_t>(k_cache->shape[2]), k->dtype,
                       k_cache->dtype, o.k_scale, o.v_scale, o.stream);
}

int pa_decode_t(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                const pa_tensor* block_tables, const pa_tensor* seq_lens, float scale, int32_t block_size,
                const pa_opts* opts) {
    static const char* fn = "pa_decode_t";
    pagedkv::clear_error();
    const pa_opts none{};
    const pa_opts& o = opts ? *opts : none;
    if (int rc = check_view(out, 3, fn, "out")) return rc;
    if (int rc = check_view(q, 3, fn, "q")) return rc;
    if (int rc = check_view(k_cache, 4, fn, "k_cache")) return rc;
    if (int rc = check_view(v_cache, 4, fn, "v_cache")) return rc;
    if (int rc = check_view(block_tables, 2, fn, "block_tables")) return rc;
    if (int rc = check_view(seq_lens, 1, fn, "seq_lens")) return rc;
    if (int rc = check_dtype(block_tables, PA_DTYPE_I32, fn, "block_tables")) return rc;
    if (int rc = check_dtype(seq_lens, PA_DTYPE_I32, fn, "seq_lens")) return rc;
    if (!same_shape(out, q) || out->dtype != q->dtype) return fail(PA_ERR_INVALID, "%s: out and q differ in shape or dtype", fn);
    if (!same_shape(k_cache, v_cache) || k_cache->dtype != v_cache->dtype)
        return fail(PA_ERR_INVALID, "%s: k_cache and v_cache differ in shape or dtype", fn);
    const int64_t B = q->shape[0], Hq = q->shape[1], d = q->shape[2];
    const int64_t N = k_cache->shape[0], Hkv = k_cache->shape[1], bs = k_cache->shape[2];
    if (k_cache->shape[3] != d)
        return fail(PA_ERR_INVALID, "%s: head_dim %lld of q, %lld of the cache", fn, (long long)d, (long long)k_cache->shape[3]);
    if (bs != block_size)
        return fail(PA_ERR_INVALID, "%s: block_size %d but the cache holds %lld rows per block", fn, block_size, (long long)bs);
    if (Hkv <= 0 || Hq % Hkv != 0)
        return fail(PA_ERR_INVALID, "%s: %lld q heads not a multiple of %lld KV heads", fn, (long long)Hq, (long long)Hkv);
    if (block_tables->shape[0] != B || seq_lens->shape[0] != B)
        return fail(PA_ERR_INVALID, "%s: %lld requests in q, %lld table rows, %lld lengths", fn, (long long)B,
                    (long long)block_tables->shape[0], (long long)seq_lens->shape[0]);
    if (B > 0x7fffffff || Hq > 0x7fffffff || d > 0x7fffffff || block_tables->shape[1] > 0x7fffffff)
        return fail(PA_ERR_INVALID, "%s: sizes beyond int32", fn);
    const int64_t max_blocks = block_tables->shape[1];
    const int32_t max_seq_len = o.max_seq_len > 0 ? o.max_seq_len : narrow(max_blocks * bs);
    return pa_decode(out->data, q->data, k_cache->data, v_cache->data, static_cast<const int32_t*>(block_tables->data),
                     static_cast<const int32_t*>(seq_lens->data), scale, block_size, static_cast<int32_t>(B),
                     static_cast<int32_t>(Hq), static_cast<int32_t>(Hkv), static_cast<int32_t>(d), N,
                     static_cast<int32_t>(max_blocks), max_seq_len, q->dtype, k_cache->dtype, o.k_scale, o.v_scale,
                     o.workspace, o.workspace_bytes, o.partition_tokens, o.stream);
}

}  // extern "C"
