/* x86 BMI2 parallel bit extract / deposit, used only to pin the oracle's
 * bit-at-a-time extract and deposit against the ISA's own definition. */
#include <stdint.h>
#include <immintrin.h>
uint64_t ref_pext(uint64_t v, uint64_t m) { return _pext_u64(v, m); }
uint64_t ref_pdep(uint64_t v, uint64_t m) { return _pdep_u64(v, m); }
