// gdn_prefill_inst.hip -- one (element type, chunk size) instantiation of the
// chunked prefill's preparation and scan kernels (gdn_prefill.hpp), for both
// gate types. The build compiles this file once per pair, with
// GDN_INST_BF16 (1: bf16 I/O, 0: fp32 I/O) and GDN_INST_CHUNK (16, 32, 64)
// defined, so that the six instantiations compile in parallel.
#include "gdn_prefill.hpp"

// Compiled without the two macros the file is empty.
#if defined(GDN_INST_BF16) && defined(GDN_INST_CHUNK)

namespace gdn {

#if GDN_INST_BF16
typedef bf16 InstElem;
#else
typedef float InstElem;
#endif

GDN_PREFILL_INST_DECL(GDN_INST_BF16, GDN_INST_CHUNK) {
    return A.gate_bf16 ? launch_prefill_c<InstElem, bf16, GDN_INST_CHUNK>(A, st)
                       : launch_prefill_c<InstElem, float, GDN_INST_CHUNK>(A, st);
}

}  // namespace gdn

#endif
