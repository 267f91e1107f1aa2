"""Float64 CPU oracle for GPTQ layer-wise weight quantization.

TEST INFRASTRUCTURE. Nothing in the product library imports, links or calls
this package; only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may use it. It shares no code, tables or helpers with the HIP
library: both sides receive the same seeded inputs from ``synth`` and nothing
else.

Modules
-------
gptq_f64   the method itself (Hessian, damping/ordering, the O1 and O2 sweeps,
           round-to-nearest, brute force, layer error)
packing    the LSB-first code bitstream and its inverse
dequant    the dequantising product Y = X W_hat^T of a packed layer
eora       the EoRA low-rank adapter of the compression error
intrinsic  OLrC / Bid-Up refinement of a low-precision plus low-rank layer
memory     storage accounting used by the pages' worked examples

Every function names the passage of the pages it follows. The pages are:
  [GPTQ]   "GPTQ" (wikiprompt.org), sections "Enfoque Técnico",
           "Rendimiento y Precisión"
  [BAL]    "El balance de errores de la inferencia de pocos bits"
           (auturnal.com), sections 1-6 and "Ejemplo resuelto"
  [GIL]    "Resumen Técnico: GPTQ-intrinsic LoRA" (gist.science 2606.01412),
           "Declaración del Problema", "Metodología" items 2 and 4
  [EORA]   "Aumento de la precisión de LLM de 2 bits con EoRA" (7minutos.es),
           section "Bucear en el espacio propio en busca de un adaptador"
"""
