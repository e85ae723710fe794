/* Compile-time and layout checks of the core C ABI of libspecverify: the
 * entry points sv_verify and sv_vat_labels, their workspace queries and
 * descriptors, sv_status_str, sv_abi_version and the seven core status codes,
 * as a C caller written against that contract sees them.  Built by
 * tests/test_api_host.py with gcc -std=c11 -Werror; a changed prototype or
 * code fails the build, a changed layout fails the test. */
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

_Static_assert(SV_OK == 0, "SV_OK");
_Static_assert(SV_ERR_NULL_ARG == 1, "SV_ERR_NULL_ARG");
_Static_assert(SV_ERR_BAD_SHAPE == 2, "SV_ERR_BAD_SHAPE");
_Static_assert(SV_ERR_BAD_DTYPE == 3, "SV_ERR_BAD_DTYPE");
_Static_assert(SV_ERR_BAD_TEMPERATURE == 4, "SV_ERR_BAD_TEMPERATURE");
_Static_assert(SV_ERR_WORKSPACE_TOO_SMALL == 5, "SV_ERR_WORKSPACE_TOO_SMALL");
_Static_assert(SV_ERR_HIP == 6, "SV_ERR_HIP");
_Static_assert(SV_F32 == 0 && SV_BF16 == 1, "sv_dtype");
_Static_assert(SV_DRAFT_LOGITS == 0 && SV_DRAFT_ONEHOT == 1, "sv_draft_kind");

typedef size_t (*verify_ws_fn)(const sv_verify_desc*);
typedef sv_status (*verify_fn)(const sv_verify_desc*, const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                               int32_t* out_tokens, float* probs_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);
typedef size_t (*vat_ws_fn)(const sv_vat_desc*);
typedef sv_status (*vat_fn)(const sv_vat_desc*, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                            int32_t* first_reject, float* weights, float* probs_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
typedef const char* (*status_str_fn)(sv_status);
typedef int (*abi_version_fn)(void);

/* Taking each entry point's address as the contract's pointer type is what
 * -Werror turns into a prototype check. */
const void* contract_entry_points(int i) {
    static const verify_ws_fn a = sv_verify_workspace_bytes;
    static const verify_fn b = sv_verify;
    static const vat_ws_fn c = sv_vat_workspace_bytes;
    static const vat_fn d = sv_vat_labels;
    static const status_str_fn e = sv_status_str;
    static const abi_version_fn f = sv_abi_version;
    switch (i) {
        case 0: return (const void*)&a;
        case 1: return (const void*)&b;
        case 2: return (const void*)&c;
        case 3: return (const void*)&d;
        case 4: return (const void*)&e;
        default: return (const void*)&f;
    }
}

/* sizeof and field offsets of both descriptors, in declaration order:
 * out[0..6] sv_verify_desc (size, B, k, V, dtype, draft_kind, temperature),
 * out[7..13] sv_vat_desc (size, N, k, V, dtype, temperature, decay). */
void contract_layout(int64_t* out) {
    out[0] = (int64_t)sizeof(sv_verify_desc);
    out[1] = (int64_t)offsetof(sv_verify_desc, B);
    out[2] = (int64_t)offsetof(sv_verify_desc, k);
    out[3] = (int64_t)offsetof(sv_verify_desc, V);
    out[4] = (int64_t)offsetof(sv_verify_desc, dtype);
    out[5] = (int64_t)offsetof(sv_verify_desc, draft_kind);
    out[6] = (int64_t)offsetof(sv_verify_desc, temperature);
    out[7] = (int64_t)sizeof(sv_vat_desc);
    out[8] = (int64_t)offsetof(sv_vat_desc, N);
    out[9] = (int64_t)offsetof(sv_vat_desc, k);
    out[10] = (int64_t)offsetof(sv_vat_desc, V);
    out[11] = (int64_t)offsetof(sv_vat_desc, dtype);
    out[12] = (int64_t)offsetof(sv_vat_desc, temperature);
    out[13] = (int64_t)offsetof(sv_vat_desc, decay);
}
